"""Pins for the oracle's RoPE: closed forms and invariants that hold for the textbook definition."""
import math

import numpy as np

THETA = 10000.0


def test_single_pair_closed_form(orc):
    # one pair, j = 0: frequency theta^0 = 1, so position p rotates by p radians
    for p in [0, 1, 7, 1000, (1 << 20) + 12345]:
        v = orc.rope(np.array([0.3, -1.7]), 2, THETA, p)
        c, s = math.cos(p), math.sin(p)
        assert np.allclose(v, [0.3 * c + 1.7 * s, 0.3 * s - 1.7 * c], atol=1e-12)


def test_pair_frequencies(orc):
    R = 16
    for j in range(R // 2):
        e = np.zeros(R)
        e[2 * j] = 1.0
        v = orc.rope(e, R, THETA, 3)
        ang = math.atan2(v[2 * j + 1], v[2 * j])
        want = math.remainder(3 * THETA ** (-2 * j / R), 2 * math.pi)
        assert abs(ang - want) < 1e-12
        others = np.delete(v, [2 * j, 2 * j + 1])
        assert np.all(others == 0)


def test_only_tail_rotates_and_pair_norms(orc):
    rs = np.random.default_rng(0)
    v = rs.standard_normal(128)
    r = orc.rope(v, 32, THETA, 777)
    assert np.array_equal(r[:96], v[:96])
    n0 = np.hypot(v[96::2], v[97::2])
    n1 = np.hypot(r[96::2], r[97::2])
    assert np.allclose(n0, n1, rtol=1e-13)


def test_inverse_identity_and_pos_zero(orc):
    rs = np.random.default_rng(1)
    v = rs.standard_normal(512)
    assert np.array_equal(orc.rope(v, 64, THETA, 0), v)
    for p in [1, 129, 131072, 1 << 20]:
        back = orc.rope(orc.rope(v, 64, THETA, p), 64, THETA, -p)
        assert np.allclose(back, v, atol=1e-12)


def test_relative_position(orc):
    rs = np.random.default_rng(2)
    u, v = rs.standard_normal(512), rs.standard_normal(512)
    base = np.dot(orc.rope(u, 64, THETA, 1000), orc.rope(v, 64, THETA, 900))
    for shift in [128, 4096, 1 << 20]:
        d = np.dot(orc.rope(u, 64, THETA, 1000 + shift), orc.rope(v, 64, THETA, 900 + shift))
        assert abs(d - base) < 1e-9

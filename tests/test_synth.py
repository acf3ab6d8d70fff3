"""The seeded generator: tensor arithmetic equals exact integer SplitMix64."""
import math

import numpy as np
import torch

from synth import rng, workloads


def _ref_bits(seed, tid, i):
    key = rng.stream_key(seed, tid)
    return rng.mix64_int(key + (i + 1) * rng.GAMMA)


def test_bits_match_exact_integers():
    for seed, tid in [(0, 1), (3, 10), (123456, 7)]:
        b = rng.bits64(seed, tid, 1000, 300)
        got = [int(v) & rng.MASK64 for v in b.tolist()]
        want = [_ref_bits(seed, tid, 1000 + i) for i in range(300)]
        assert got == want


def test_splitmix_known_value():
    # SplitMix64 seeded with 0 (state += gamma, then mix) yields 0xE220A8397B1DCDAF first.
    assert rng.mix64_int(rng.GAMMA) == 0xE220A8397B1DCDAF


def test_uniform_and_normal_from_bits():
    u = rng.uniform(5, 2, 64)
    for i in range(64):
        assert u[i].item() == (_ref_bits(5, 2, i) >> 11) * 2.0 ** -53
    z = rng.normal(5, 2, 16, dtype=torch.float64)
    for i in range(16):
        u1 = (_ref_bits(5, 2, 2 * i) >> 11) * 2.0 ** -53
        u2 = (_ref_bits(5, 2, 2 * i + 1) >> 11) * 2.0 ** -53
        assert abs(z[i].item() - math.sqrt(-2 * math.log(1 - u1)) * math.cos(2 * math.pi * u2)) < 1e-12


def test_offsets_regenerate_slices():
    full = rng.normal_bf16(1, 3, 5000)
    part = rng.normal_bf16(1, 3, 1000, start=2500)
    assert torch.equal(full[2500:3500], part)


def test_distribution_and_permutation():
    z = rng.normal(0, 1, 200000).numpy()
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    p = rng.permutation(0, 11, 4096).numpy()
    assert np.array_equal(np.sort(p), np.arange(4096))


def test_workload_shapes():
    w = workloads.c4a_decode()
    assert w.max_blocks == 513 and w.num_q == 16 and int(w.query_positions()[0]) == 131072
    t = workloads.tiny()
    assert t.num_q == 16 and list(t.query_positions()[:2]) == [1008, 1009]
    pf = workloads.prefill()
    assert pf.num_q == 8192 and int(pf.query_positions()[-1]) == 65536 + 8191

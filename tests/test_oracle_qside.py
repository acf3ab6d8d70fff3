"""Pins for the oracle's query-side step: per-head Q RMSNorm + Q RoPE at the
token's position, beside the raw-key RoPE + insert ([Notes] 融合 3：Q Norm +
KV RoPE + K Insert).  Expected values come from a hand-worked example, closed
forms (a constant head normalises to +-1), the rotation's invariants (norm,
identity at position 0, logits that depend on the query-key distance only)
and consistency with the separately pinned RoPE and raw insert."""
import math

import numpy as np
import pytest
import torch

from tests.util import bf16_np, bf16_to_f64, block_table, gather_rows, randn_bf16, rand_u

THETA = 10000.0


def bf16_rne(v) -> np.ndarray:
    """Round fp64 values to bf16 bits with torch's conversion (independent of the oracle)."""
    return bf16_np(torch.tensor(np.asarray(v, np.float64), dtype=torch.float64).to(torch.bfloat16))


def one_seq(orc, q, x, start, dim, rope_dims, gain=None, eps=1e-6, seed=0):
    """q [n][H][dim], x [n][dim] (bf16 bits) as one chunk at start..start+n-1."""
    n = q.shape[0]
    mb = (start + n + 255) // 256 + 1
    bt = block_table(seed, 1, mb, extra_pages=2)
    pool = orc.HostPool(1, 1, dim, rope_dims, THETA, orc.BF16, mb + 2, state=False)
    out, f = orc.q_norm_rope_insert(pool, bt, [start], [0, n], x, q, gain, eps)
    assert f == 0
    return out, pool, bt


def test_hand_worked_example(orc):
    # D = 4, one rotated pair (dims 2, 3) at frequency theta^0 = 1; token at position 1.
    # q = (1, -1, 2, 0): mean square 6/4 = 1.5, so y = q / sqrt(1.5 + 1e-6); the pair
    # (2, 0)/rms turns by 1 radian.
    q = bf16_rne([[[1.0, -1.0, 2.0, 0.0]]])
    x = bf16_rne([[0.5, 0.25, -1.0, 3.0]])
    out, pool, bt = one_seq(orc, q, x, 1, 4, 2)
    rms = math.sqrt(1.5 + 1e-6)
    want = [1 / rms, -1 / rms, 2 * math.cos(1.0) / rms, 2 * math.sin(1.0) / rms]
    assert np.array_equal(out[0, 0], bf16_rne(want))
    # the raw key row: no norm, the same rotation: (-1, 3) turns by 1 radian
    row = gather_rows(pool.rows, bt, 0, 1, 1, 1).view(np.uint16)[0]
    c, s = math.cos(1.0), math.sin(1.0)
    assert np.array_equal(row, bf16_rne([0.5, 0.25, -c - 3 * s, -s + 3 * c]))


@pytest.mark.parametrize("c", [-3.5, 0.125, 40.0])
def test_constant_head_normalises_to_unit(orc, c):
    # q_h = c * 1: mean square c^2, so y = c / sqrt(c^2 + eps) = sign(c) to bf16 precision
    D, H = 64, 3
    q = np.broadcast_to(bf16_rne([c]), (2, H, D)).copy()
    x = np.zeros((2, D), np.uint16)
    out, _, _ = one_seq(orc, q, x, 0, D, 0)
    assert np.all(bf16_to_f64(out) == math.copysign(1.0, c))


def test_zero_head_stays_zero(orc):
    D = 32
    q = np.zeros((1, 2, D), np.uint16)
    out, _, _ = one_seq(orc, q, np.zeros((1, D), np.uint16), 9, D, 16)
    assert not bf16_to_f64(out).any()


def test_gain_is_per_dim_and_shared_by_heads(orc):
    D, H, n = 64, 4, 3
    q = randn_bf16(3, 1, (n, H, D))
    x = randn_bf16(3, 2, (n, D))
    g = np.ones(D, np.float32)
    g[5], g[40] = 2.0, 0.0   # a power of two scales exactly through bf16 rounding
    plain, _, _ = one_seq(orc, q, x, 0, D, 0)
    gained, _, _ = one_seq(orc, q, x, 0, D, 0, gain=g)
    a, b = bf16_to_f64(plain), bf16_to_f64(gained)
    assert np.array_equal(b[..., 5], 2.0 * a[..., 5])
    assert not b[..., 40].any()
    keep = [d for d in range(D) if d not in (5, 40)]
    assert np.array_equal(a[..., keep], b[..., keep])


def test_rotation_only_on_tail_preserves_norm(orc):
    D, R, H, n = 128, 32, 4, 5
    q = randn_bf16(4, 1, (n, H, D))
    x = randn_bf16(4, 2, (n, D))
    flat, _, _ = one_seq(orc, q, x, 300, D, 0)
    rot, _, _ = one_seq(orc, q, x, 300, D, R)
    assert np.array_equal(rot[..., :D - R], flat[..., :D - R])
    f, r = bf16_to_f64(flat[..., D - R:]), bf16_to_f64(rot[..., D - R:])
    pf = np.hypot(f[..., 0::2], f[..., 1::2])
    pr = np.hypot(r[..., 0::2], r[..., 1::2])
    assert np.allclose(pr, pf, rtol=2 ** -7, atol=1e-6)
    assert not np.allclose(r, f, atol=1e-2)
    # RMSNorm with unit gain: every head has mean square ~1 (eps is negligible here)
    ms = np.mean(bf16_to_f64(rot) ** 2, axis=-1)
    assert np.allclose(ms, 1.0, rtol=2 ** -6)


def test_position_is_start_plus_offset(orc):
    # token j of a chunk starting at `start` is rotated at start + j: the unrotated
    # output, rotated by the pinned RoPE at that position, gives the same bf16 values
    D, R, H, n, start = 64, 32, 2, 4, 1021
    q = randn_bf16(5, 1, (n, H, D))
    x = randn_bf16(5, 2, (n, D))
    flat, _, _ = one_seq(orc, q, x, start, D, 0)
    rot, _, _ = one_seq(orc, q, x, start, D, R)
    for j in range(n):
        for h in range(H):
            # the flat output is the bf16 of the normed head; rotating that rounded value
            # differs from rotating the exact one by at most ~2 bf16 ulps
            v = orc.rope(bf16_to_f64(flat[j, h]), R, THETA, start + j)
            assert np.allclose(bf16_to_f64(rot[j, h]), v, rtol=2 ** -6, atol=2 ** -7)
    # the position is not j alone
    v0 = orc.rope(bf16_to_f64(flat[1, 0]), R, THETA, 1)
    assert not np.allclose(bf16_to_f64(rot[1, 0]), v0, rtol=2 ** -6, atol=2 ** -7)


def test_logit_depends_on_query_key_distance(orc):
    # q rotated at p and a raw key rotated at t: <q_out, k> depends on p - t only
    D, R = 128, 64
    q = randn_bf16(6, 1, (1, 1, D))
    x = randn_bf16(6, 2, (1, D))
    logits = []
    for p, t in [(900, 880), (900 + 4321, 880 + 4321), (20, 0)]:
        qo, _, _ = one_seq(orc, q, x, p, D, R)
        _, pool, bt = one_seq(orc, q, x, t, D, R)
        k = bf16_to_f64(gather_rows(pool.rows, bt, 0, 1, t, 1).view(np.uint16)[0])
        logits.append(float(bf16_to_f64(qo[0, 0]) @ k))
    assert abs(logits[0] - logits[1]) < 0.05 and abs(logits[0] - logits[2]) < 0.05
    # a different distance gives a different logit
    qo, _, _ = one_seq(orc, q, x, 905, D, R)
    _, pool, bt = one_seq(orc, q, x, 880, D, R)
    k = bf16_to_f64(gather_rows(pool.rows, bt, 0, 1, 880, 1).view(np.uint16)[0])
    assert abs(float(bf16_to_f64(qo[0, 0]) @ k) - logits[0]) > 0.05


def test_raw_insert_equals_ratio1_compress_insert(orc):
    D, R, H = 64, 16, 2
    starts, lens = [0, 250, 4000], [3, 0, 9]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    n = int(cu[-1])
    q = randn_bf16(8, 1, (n, H, D))
    x = randn_bf16(8, 2, (n, D))
    mb = 17
    bt = block_table(8, 3, mb, extra_pages=1)
    a = orc.HostPool(1, 1, D, R, THETA, orc.BF16, 3 * mb + 1, state=False)
    b = orc.HostPool(1, 1, D, R, THETA, orc.BF16, 3 * mb + 1, state=False)
    _, f = orc.q_norm_rope_insert(a, bt, starts, cu, x, q)
    assert f == 0
    assert orc.compress_insert(b, bt, starts, cu, x) == 0
    assert np.array_equal(a.rows, b.rows)


def test_chunking_and_batching_do_not_change_queries(orc):
    # three sequences in one call equal each sequence alone, fed in two chunks
    D, R, H = 64, 32, 3
    starts, lens = [7, 0, 1000], [5, 1, 6]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    n = int(cu[-1])
    q = randn_bf16(9, 1, (n, H, D))
    x = randn_bf16(9, 2, (n, D))
    g = rand_u(9, 3, (D,), 0.5, 1.5).astype(np.float32)
    bt = block_table(9, 3, 6)
    pool = orc.HostPool(1, 1, D, R, THETA, orc.BF16, 18, state=False)
    together, f = orc.q_norm_rope_insert(pool, bt, starts, cu, x, q, g)
    assert f == 0
    for s in range(3):
        lo, hi = int(cu[s]), int(cu[s + 1])
        half = (hi - lo) // 2
        parts = []
        for a, b in [(lo, lo + half), (lo + half, hi)]:
            o, _, _ = one_seq(orc, q[a:b], x[a:b], starts[s] + a - lo, D, R, gain=g)
            parts.append(o)
        assert np.array_equal(np.concatenate(parts), together[lo:hi])


def test_unmapped_page_counts_a_fault_but_queries_are_written(orc):
    D, H = 32, 2
    q = randn_bf16(10, 1, (2, H, D))
    x = randn_bf16(10, 2, (2, D))
    bt = np.array([[0, -1]], np.int32)
    pool = orc.HostPool(1, 1, D, 0, THETA, orc.BF16, 2, state=False)
    out, f = orc.q_norm_rope_insert(pool, bt, [255], [0, 2], x, q)
    assert f == 1                     # token 256 falls in the unmapped block
    assert np.all(np.abs(np.mean(bf16_to_f64(out) ** 2, axis=-1) - 1.0) < 2 ** -6)

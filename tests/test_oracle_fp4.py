"""Pins for the oracle's fp4 rows (the fp4 index cache): OCP MXFP4, i.e. E2M1
elements with one E8M0 power-of-two scale per 32 elements.  Expected values
come from the format's definition (code table, tie rule, scale rule), worked
out by hand here, not from the oracle's encoder."""
import math

import numpy as np
import pytest

from tests.test_oracle_compress import run
from tests.util import fp4_rows, randn_bf16, randn_f32

# E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is
# subnormal (0 or 0.5); no infinities or NaN.
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def elem(codes, i):
    return (int(codes[i // 2]) >> (4 * (i & 1))) & 15


def test_e2m1_decode_all_codes(orc):
    for c in range(16):
        got = orc.e2m1_to_f64(c)
        sign = -1.0 if c & 8 else 1.0
        assert got == sign * E2M1[c & 7]
        assert math.copysign(1.0, got) == sign  # code 8 is -0


# (value, code): midpoints between neighbours go to the code with mantissa bit 0
TIES = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)]
# off-midpoint values and saturation
NEAR = [(0.0, 0), (0.24, 0), (0.26, 1), (0.74, 1), (0.76, 2), (1.3, 3), (1.7, 3), (2.4, 4), (2.6, 5), (3.4, 5),
        (3.6, 6), (4.9, 6), (5.1, 7), (6.0, 7), (7.99, 7), (1e6, 7)]


@pytest.mark.parametrize("v,c", TIES + NEAR)
def test_e2m1_rounding(orc, v, c):
    assert orc.f64_to_e2m1(v) == c
    assert orc.f64_to_e2m1(-v) == 8 | c


def test_e2m1_representable_values_roundtrip(orc):
    for c in range(16):
        assert orc.f64_to_e2m1(orc.e2m1_to_f64(c)) == c


def test_mxfp4_scale_rule(orc):
    # X = 2^(floor(log2 amax) - 2): amax in [4, 8) gives X = 1 (code 127)
    y = np.zeros(32)
    y[3], y[4], y[5] = 6.0, -0.5, 2.5
    codes, sc = orc.mxfp4_block(y)
    assert sc == 127 and elem(codes, 3) == 7 and elem(codes, 4) == 9 and elem(codes, 5) == 4
    assert all(elem(codes, i) in (0, 8) for i in range(32) if i not in (3, 4, 5))
    # amax 7.9: still X = 1, the maximum saturates to 6
    y[3] = 7.9
    codes, sc = orc.mxfp4_block(y)
    assert sc == 127 and elem(codes, 3) == 7
    # amax 1: floor(log2) = 0, X = 1/4, 1.0 -> 4 (code 6); 0.3 -> 1.2 -> 1.0 (code 2)
    y = np.zeros(32)
    y[0], y[31] = 1.0, 0.3
    codes, sc = orc.mxfp4_block(y)
    assert sc == 125 and elem(codes, 0) == 6 and elem(codes, 31) == 2
    # amax 0.3: floor(log2 0.3) = -2, X = 2^-4, 0.3 * 16 = 4.8 -> 4 (code 6)
    y = np.zeros(32)
    y[7] = -0.3
    codes, sc = orc.mxfp4_block(y)
    assert sc == 123 and elem(codes, 7) == 8 | 6
    # an all-zero block: scale code 0, codes 0
    codes, sc = orc.mxfp4_block(np.zeros(32))
    assert sc == 0 and not codes.any()
    # tiny amax: the exponent clamps at -127 (code 0)
    y = np.zeros(32)
    y[0] = 2.0 ** -126
    codes, sc = orc.mxfp4_block(y)
    assert sc == 0 and elem(codes, 0) == 4  # 2^-126 / 2^-127 = 2


def test_mxfp4_representable_blocks_roundtrip(orc):
    rng = np.random.default_rng(3)
    for _ in range(200):
        k = int(rng.integers(-20, 20))
        c = rng.integers(0, 16, 32)
        c[int(rng.integers(0, 32))] = int(rng.choice([6, 7, 14, 15]))  # a magnitude of 4 or 6 sets X = 2^k
        vals = np.array([(-1.0 if ci & 8 else 1.0) * E2M1[ci & 7] for ci in c]) * 2.0 ** k
        codes, sc = orc.mxfp4_block(vals)
        assert sc == k + 127
        back = np.array([orc.e2m1_to_f64(elem(codes, i)) for i in range(32)]) * 2.0 ** (sc - 127)
        assert np.array_equal(back, vals)


def _err_bound(y, X):
    """The format's element error at block scale X: half the grid spacing at |y|/X, or the
    distance to 6 once saturated; plus the fp32 rounding of the input."""
    r = np.abs(y) / X
    half = np.where(r <= 2, 0.25, np.where(r <= 4, 0.5, np.where(r <= 6, 1.0, r - 6.0)))
    return X * half + np.abs(y) * 2.0 ** -24


def test_mxfp4_error_bound_random(orc):
    rng = np.random.default_rng(5)
    for scale in (1e-3, 1.0, 37.0):
        for _ in range(100):
            y = rng.standard_normal(32) * scale
            codes, sc = orc.mxfp4_block(y)
            X = 2.0 ** (sc - 127)
            assert X == 2.0 ** (math.floor(math.log2(np.abs(y.astype(np.float32)).max())) - 2)
            back = np.array([orc.e2m1_to_f64(elem(codes, i)) for i in range(32)]) * X
            assert np.all(np.abs(back - y) <= _err_bound(y, X))


def test_fp4_row_layout(orc):
    assert orc.row_bytes(128, orc.FP4) == 68 and orc.row_bytes(32, orc.FP4) == 17
    # one 64-dim row: codes (element 2i low nibble of byte i), then 2 E8M0 bytes
    row = np.zeros(34, np.uint8)
    row[0] = 0x71          # elements 0, 1 = 0.5, 6
    row[31] = 0xA0         # elements 62, 63 = 0, -1
    row[32], row[33] = 127, 130
    v = orc.decode_rows(row[None, :], 64, orc.FP4)[0]
    assert v[0] == 0.5 and v[1] == 6.0 and v[62] == 0.0 and v[63] == -8.0
    assert np.count_nonzero(v) == 3


def test_fp4_compressor_rows(orc):
    x = randn_bf16(7, 1, (1024, 64))
    lg = randn_f32(7, 2, (1024, 2)).astype(np.float32)
    y32, _, _ = run(orc, x, lg, 4, 2, rope_dims=16, dtype=orc.F32)
    deq, _, _ = run(orc, x, lg, 4, 2, rope_dims=16, dtype=orc.FP4)
    for b in range(2):
        blk = y32[:, 32 * b:32 * b + 32]
        X = 2.0 ** (np.floor(np.log2(np.abs(blk).max(axis=1))) - 2)
        assert np.all(np.abs(deq[:, 32 * b:32 * b + 32] - blk) <= _err_bound(blk, X[:, None]))


def test_fp4_index_pool_scores_as_its_values(orc):
    """The indexer over an fp4 pool equals the indexer over a bf16 pool holding the
    decoded values (E2M1 values times a power of two are exact in bf16)."""
    from tests.test_oracle_index import THETA as ITHETA, bf16, index_pool
    from tests.util import bf16_to_f64, block_table, rand_u, scatter_rows
    n, d, nq, H = 300, 64, 5, 4
    vals = np.random.default_rng(11).standard_normal((n, d)) * 3.0
    rows = fp4_rows(orc, vals)
    deq = orc.decode_rows(rows, d, orc.FP4)
    assert np.array_equal(bf16_to_f64(bf16(deq)), deq)
    mb = (4 * n + 255) // 256 + 1
    bt4 = block_table(5, 1, mb, extra_pages=2)
    pool4 = orc.HostPool(4, 2, d, 0, ITHETA, orc.FP4, mb + 2)
    scatter_rows(pool4.rows, bt4, 0, 4, rows)
    pool16, bt16 = index_pool(orc, bf16(deq))
    q = randn_bf16(11, 2, (nq, H, d))
    w = rand_u(11, 3, (nq, H)).astype(np.float32)
    pos = np.array([1200, 999, 640, 37, 3], np.int64)
    seqs = np.zeros(nq, np.int32)
    a = orc.index_topk(pool4, bt4, seqs, pos, q, w, 48, want_scores=True, max_cand=n)
    b = orc.index_topk(pool16, bt16, seqs, pos, q, w, 48, want_scores=True, max_cand=n)
    assert a[3] == 0 and b[3] == 0
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])

"""Pins for the oracle's compressor + RMSNorm + RoPE + paged insert.

Window definitions ([Notes] 数学附录精要): c4a entry i covers tokens
[4i-4, 4i+3] (negative positions absent) and is rotated at 4i; c128a entry i
covers [128i, 128i+127] and is rotated at 128i.
"""
import numpy as np
import pytest

from tests.util import bf16_to_f64, block_table, gather_rows, randn_bf16, randn_f32

THETA = 10000.0


def run(orc, x, logits, ratio, coff, rope_dims=0, dtype=None, gain=None, chunks=None, seed=0, eps=1e-6):
    """Compress one sequence x [T][D] (bf16 bits); returns (decoded entries [T//r][D], pool, bt)."""
    dtype = orc.BF16 if dtype is None else dtype
    T, D = x.shape
    mb = (T + 255) // 256
    bt = block_table(seed, 1, mb, extra_pages=3)
    pool = orc.HostPool(ratio, coff, D, rope_dims, THETA, dtype, mb + 3)
    chunks = chunks or [T]
    t0 = 0
    for n in chunks:
        f = orc.compress_insert(pool, bt, [t0], [0, n], x[t0:t0 + n], None if logits is None else logits[t0:t0 + n],
                                gain, eps)
        assert f == 0
        t0 += n
    assert t0 == T
    rows = gather_rows(pool.rows, bt, 0, ratio, 0, T // ratio)
    return orc.decode_rows(rows, D, dtype), pool, bt


def rms_normalise(u, eps=1e-6):
    return u / np.sqrt(np.mean(u * u, axis=-1, keepdims=True) + eps)


@pytest.fixture(scope="module")
def seq():
    x = randn_bf16(7, 1, (1024, 64))
    return x, bf16_to_f64(x)


def test_c4a_uniform_weights_give_window_mean(orc, seq):
    x, xf = seq
    y, _, _ = run(orc, x, np.zeros((1024, 2), np.float32), 4, 2)
    assert y.shape == (256, 64)
    for i in range(256):
        lo = max(0, 4 * i - 4)
        want = rms_normalise(xf[lo:4 * i + 4].mean(0))
        assert np.allclose(y[i], want, rtol=8e-3, atol=8e-3), i


def test_c128a_uniform_weights_give_window_mean(orc, seq):
    x, xf = seq
    y, _, _ = run(orc, x, np.zeros((1024, 1), np.float32), 128, 1)
    assert y.shape == (8, 64)
    for i in range(8):
        want = rms_normalise(xf[128 * i:128 * i + 128].mean(0))
        assert np.allclose(y[i], want, rtol=8e-3, atol=8e-3)


def test_logit_columns(orc, seq):
    # column 0 is the logit a token carries in the lookback half of the next entry,
    # column 1 the one it carries in its own entry: +40 on column 0 everywhere makes
    # entry i >= 1 the mean of tokens 4i-4..4i-1, and entry 0 (no lookback) the mean of 0..3
    x, xf = seq
    lg = np.zeros((1024, 2), np.float32)
    lg[:, 0] = 40.0
    y, _, _ = run(orc, x, lg, 4, 2)
    assert np.allclose(y[0], rms_normalise(xf[0:4].mean(0)), rtol=8e-3, atol=8e-3)
    for i in range(1, 256):
        assert np.allclose(y[i], rms_normalise(xf[4 * i - 4:4 * i].mean(0)), rtol=8e-3, atol=8e-3)


def test_single_dominant_logit_selects_one_token(orc, seq):
    x, xf = seq
    lg = np.zeros((1024, 2), np.float32)
    lg[4 * 10 + 2, 1] = 40.0        # token 42, own half of entry 10
    y, _, _ = run(orc, x, lg, 4, 2)
    assert np.allclose(y[10], rms_normalise(xf[42]), rtol=8e-3, atol=8e-3)


def test_softmax_weights_closed_form(orc, seq):
    x, xf = seq
    lg = randn_f32(7, 2, (1024, 2)).astype(np.float32)
    y, _, _ = run(orc, x, lg, 4, 2)
    for i in [0, 1, 77, 255]:
        ts = [t for t in range(4 * i - 4, 4 * i + 4) if t >= 0]
        col = [0 if t < 4 * i else 1 for t in ts]
        l = np.array([lg[t, c] for t, c in zip(ts, col)], np.float64)
        w = np.exp(l - l.max())
        w /= w.sum()
        assert np.allclose(y[i], rms_normalise((w[:, None] * xf[ts]).sum(0)), rtol=8e-3, atol=8e-3)


def test_rms_and_scale_invariance(orc, seq):
    x, xf = seq
    lg = randn_f32(7, 2, (1024, 2)).astype(np.float32)
    y, _, _ = run(orc, x, lg, 4, 2, dtype=orc.F32)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, atol=1e-5)
    x2 = (x.astype(np.uint32) + (1 << 7)).astype(np.uint16)  # +1 in the bf16 exponent: exact x*2
    y2, _, _ = run(orc, x2, lg, 4, 2, dtype=orc.F32)
    assert np.allclose(y, y2, atol=1e-5)
    g = np.linspace(0.5, 1.5, 64).astype(np.float32)
    yg, _, _ = run(orc, x, lg, 4, 2, dtype=orc.F32, gain=g)
    assert np.allclose(yg / g, y, atol=1e-6)


def test_rope_position_of_entries(orc, seq):
    x, _ = seq
    lg = randn_f32(7, 2, (1024, 2)).astype(np.float32)
    y0, _, _ = run(orc, x, lg, 4, 2, rope_dims=0, dtype=orc.F32)
    y1, _, _ = run(orc, x, lg, 4, 2, rope_dims=32, dtype=orc.F32)
    for i in [0, 1, 2, 100, 255]:
        back = orc.rope(y1[i], 32, THETA, -4 * i)
        assert np.allclose(back, y0[i], atol=1e-6)
    lg1 = randn_f32(7, 3, (1024, 1)).astype(np.float32)
    z0, _, _ = run(orc, x, lg1, 128, 1, rope_dims=0, dtype=orc.F32)
    z1, _, _ = run(orc, x, lg1, 128, 1, rope_dims=32, dtype=orc.F32)
    for i in range(8):
        assert np.allclose(orc.rope(z1[i], 32, THETA, -128 * i), z0[i], atol=1e-6)


def test_locality(orc, seq):
    x, _ = seq
    lg = randn_f32(7, 2, (1024, 2)).astype(np.float32)
    base, _, _ = run(orc, x, lg, 4, 2, rope_dims=16)
    base128, _, _ = run(orc, x, lg[:, :1].copy(), 128, 1, rope_dims=16)
    for t in [0, 3, 4, 517, 1023]:
        xp = x.copy()
        xp[t] = randn_bf16(8, t, (64,))
        y, _, _ = run(orc, xp, lg, 4, 2, rope_dims=16)
        changed = set(np.nonzero(np.any(y != base, axis=1))[0].tolist())
        assert changed == {i for i in (t // 4, t // 4 + 1) if i < 256}
        y128, _, _ = run(orc, xp, lg[:, :1].copy(), 128, 1, rope_dims=16)
        changed = set(np.nonzero(np.any(y128 != base128, axis=1))[0].tolist())
        assert changed == {t // 128}


@pytest.mark.parametrize("ratio,coff", [(4, 2), (128, 1)])
def test_chunked_equals_one_shot(orc, seq, ratio, coff):
    x, _ = seq
    lg = randn_f32(7, 4, (1024, coff)).astype(np.float32)
    one, p1, _ = run(orc, x, lg, ratio, coff, rope_dims=16, dtype=orc.FP8)
    rs = np.random.default_rng(ratio)
    for _ in range(3):
        cuts = np.sort(rs.choice(np.arange(1, 1024), size=9, replace=False))
        chunks = np.diff(np.concatenate([[0], cuts, [1024]])).tolist()
        ch, p2, _ = run(orc, x, lg, ratio, coff, rope_dims=16, dtype=orc.FP8, chunks=chunks)
        assert np.array_equal(one, ch)
    dec = run(orc, x, lg, ratio, coff, rope_dims=16, dtype=orc.FP8, chunks=[1] * 1024)[0]
    assert np.array_equal(one, dec)


def test_raw_rows_are_rope_at_token(orc, seq):
    x, xf = seq
    y, _, _ = run(orc, x, None, 1, 1, rope_dims=32, dtype=orc.F32)
    assert y.shape == (1024, 64)
    for t in [0, 1, 255, 256, 1023]:
        assert np.allclose(orc.rope(y[t], 32, THETA, -t), xf[t], atol=1e-6)


def test_fp8_rows(orc, seq):
    x, _ = seq
    lg = randn_f32(7, 2, (1024, 2)).astype(np.float32)
    y32, _, _ = run(orc, x, lg, 4, 2, rope_dims=16, dtype=orc.F32)
    _, pool, bt = run(orc, x, lg, 4, 2, rope_dims=16, dtype=orc.FP8)
    rows = gather_rows(pool.rows, bt, 0, 4, 0, 256)
    codes = rows[:, :64]
    scale = rows[:, 64:68].copy().view(np.float32)[:, 0].astype(np.float64)
    amax = np.abs(y32).max(axis=1)
    assert np.allclose(scale, amax / 448.0, rtol=1e-6)
    arg = np.abs(y32).argmax(axis=1)
    assert np.all((codes[np.arange(256), arg] & 0x7F) == 0x7E)   # the group max lands on +-448
    deq = orc.decode_rows(rows, 64, orc.FP8)
    # |y - s*dec(enc(y/s))| <= s * ulp/2 (ulp of e4m3 at |y/s|) up to the fp32 input rounding
    r = np.abs(y32) / scale[:, None]
    ulp = np.where(r < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(r, 1e-30))) - 3))
    assert np.all(np.abs(deq - y32) <= scale[:, None] * (ulp / 2) * (1 + 1e-6) + 1e-6)


def test_unmapped_page_counts_fault(orc, seq):
    x, _ = seq
    bt = block_table(0, 1, 4)
    bt[0, 2] = -1
    pool = orc.HostPool(4, 2, 64, 0, THETA, orc.BF16, 4)
    f = orc.compress_insert(pool, bt, [0], [0, 1024], x, np.zeros((1024, 2), np.float32))
    assert f > 0


@pytest.mark.parametrize("ratio,coff,dtype", [(4, 2, "FP8"), (128, 1, "BF16"), (1, 1, "FP8")])
def test_rows_one_by_one_equal_streaming_insert(orc, seq, ratio, coff, dtype):
    """Entries computed from explicit windows (no state, used to check sampled
    entries of large caches) are byte-identical to the streaming insert."""
    x, _ = seq
    x = np.concatenate([x, randn_bf16(7, 9, (1024, 192))], axis=1)   # D = 256 for fp8 rows
    D = x.shape[1]
    dt = getattr(orc, dtype)
    lg = None if ratio == 1 else randn_f32(7, 5, (1024, coff)).astype(np.float32)
    gain = None if ratio == 1 else np.random.default_rng(3).uniform(0.5, 1.5, D).astype(np.float32)
    T = 1024
    mb = T // 256
    bt = block_table(5, 1, mb)
    pool = orc.HostPool(ratio, coff, D, 32, THETA, dt, mb)
    assert orc.compress_insert(pool, bt, [0], [0, T], x, lg, gain) == 0
    rows = gather_rows(pool.rows, bt, 0, ratio, 0, T // ratio)
    W = coff * ratio
    ids = np.array(sorted(set([0, 1, 2, T // ratio - 1] + list(np.random.default_rng(ratio).integers(0, T // ratio, 12)))))
    xw = np.zeros((len(ids), W, D), np.uint16)
    lw = None if lg is None else np.zeros((len(ids), W, coff), np.float32)
    for m, i in enumerate(ids):
        for k in range(W):
            t = ratio * (i + 1) - W + k
            if t >= 0:
                xw[m, k] = x[t]
                if lw is not None:
                    lw[m, k] = lg[t]
    got = orc.compress_rows(ratio, coff, D, 32, THETA, dt, ids, xw, lw, gain)
    assert np.array_equal(got, rows[ids])

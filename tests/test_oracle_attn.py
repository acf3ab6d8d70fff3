"""Pins for the oracle's hybrid attention (top-k / dense compressed keys + raw window,
one softmax, K = V, inverse RoPE at the query position, output store).

The central pin is a brute-force twin: textbook masked softmax attention over
the FULL key list [all compressed entries ; all raw tokens] with an explicit
boolean mask, written here in numpy, which must equal the oracle's gather-based
result to 1e-12.
"""
import numpy as np
import pytest

from tests.util import bf16_to_f64, block_table, randn_bf16, scatter_rows

THETA = 10000.0


def make_layer(orc, seed, T, D, R, ratio, kv_dtype=None, row_dtype_f32=False):
    """One sequence of T tokens: compressed pool (ratio) + raw pool with drawn rows.

    Rows are stored directly (they stand for already-inserted cache rows).
    Returns pools, block table and the fp64 values of every stored row."""
    dt = orc.F32 if row_dtype_f32 else (orc.BF16 if kv_dtype is None else kv_dtype)
    mb = T // 256 + 1
    bt = block_table(seed, 1, mb, extra_pages=1)
    comp = orc.HostPool(ratio, 1, D, R, THETA, dt, mb + 1, state=False)
    raw = orc.HostPool(1, 1, D, R, THETA, dt, mb + 1, state=False)
    nc = T // ratio
    cv = randn_bf16(seed, 30, (nc, D))
    rv = randn_bf16(seed, 31, (T, D))
    if dt == orc.BF16:
        crow, rrow = cv.view(np.uint8).reshape(nc, -1), rv.view(np.uint8).reshape(T, -1)
    elif dt == orc.F32:
        crow = bf16_to_f64(cv).astype(np.float32).view(np.uint8).reshape(nc, -1)
        rrow = bf16_to_f64(rv).astype(np.float32).view(np.uint8).reshape(T, -1)
    else:
        crow, rrow = fp8_rows(orc, bf16_to_f64(cv)), fp8_rows(orc, bf16_to_f64(rv))
    scatter_rows(comp.rows, bt, 0, ratio, crow)
    scatter_rows(raw.rows, bt, 0, 1, rrow)
    cf = orc.decode_rows(crow, D, dt)
    rf = orc.decode_rows(rrow, D, dt)
    return comp, raw, bt, cf, rf


def fp8_rows(orc, y):
    n, D = y.shape
    out = np.empty((n, D + 4 * (D // 64)), np.uint8)
    for g in range(D // 64):
        blk = y[:, 64 * g:64 * g + 64]
        sc = (np.abs(blk).max(1) / 448.0).astype(np.float32)
        sc[sc == 0] = 1.0
        for i in range(n):
            out[i, 64 * g:64 * g + 64] = [orc.f64_to_e4m3(v / float(sc[i])) for v in blk[i]]
        out[:, D + 4 * g:D + 4 * g + 4] = sc.view(np.uint8).reshape(n, 4)
    return out


def twin(orc, q, pos, cf, rf, ratio, allowed_slots, S, R, scale):
    """Textbook masked attention over [all entries ; all raw tokens], then RoPE^-1(p)."""
    K = np.concatenate([cf, rf], 0)
    nc = cf.shape[0]
    out = np.zeros(q.shape)
    for n in range(q.shape[0]):
        p = int(pos[n])
        mask = np.zeros(K.shape[0], bool)
        for j in range(nc):
            mask[j] = ratio * (j + 1) <= p and (allowed_slots is None or j in allowed_slots[n])
        for t in range(rf.shape[0]):
            mask[nc + t] = p - S <= t <= p - 1
        if not mask.any():
            continue
        z = scale * (q[n] @ K.T)
        z[:, ~mask] = -np.inf
        a = np.exp(z - z.max(1, keepdims=True))
        a /= a.sum(1, keepdims=True)
        o = a @ K
        out[n] = np.stack([orc.rope(o[h], R, THETA, -p) for h in range(o.shape[0])])
    return out


@pytest.mark.parametrize("ratio", [4, 128])
def test_brute_force_twin(orc, ratio):
    T, D, R, H, k, S = 1024, 128, 32, 8, 16, 128
    comp, raw, bt, cf, rf = make_layer(orc, 11, T, D, R, ratio)
    pos = np.array([1, 3, 4, 127, 128, 129, 300, 1000, 1024], np.int64)
    nq = len(pos)
    q = randn_bf16(11, 40, (nq, H, D))
    qf = bf16_to_f64(q)
    if ratio == 4:
        rs = np.random.default_rng(5)
        topk = np.full((nq, k), -1, np.int32)
        for n in range(nq):
            nc = int(pos[n]) // 4
            pick = np.sort(rs.choice(nc, size=min(k, nc), replace=False)) if nc else []
            topk[n, :len(pick)] = pick
        allowed = [set(t[t >= 0].tolist()) for t in topk]
    else:
        topk, allowed = None, None
    out, _, o64, f = orc.hybrid_attn(comp, raw, bt, np.zeros(nq, np.int32), pos, q, topk=topk, k=k,
                                     swa_window=S, softmax_scale=D ** -0.5, out_dtype=orc.F32)
    assert f == 0
    want = twin(orc, qf, pos, cf, rf, ratio, allowed, S, R, D ** -0.5)
    assert np.allclose(o64, want, rtol=1e-12, atol=1e-12)
    assert np.array_equal(out, o64.astype(np.float32))


def test_single_key_closed_form(orc):
    T, D, R = 512, 128, 32
    comp, raw, bt, cf, rf = make_layer(orc, 12, T, D, R, 4)
    q = randn_bf16(12, 40, (1, 2, D))
    # p = 1: no compressed entry is visible, the window holds token 0 only
    _, _, o, _ = orc.hybrid_attn(comp, raw, bt, [0], [1], q, topk=np.full((1, 4), -1, np.int32), swa_window=128)
    for h in range(2):
        assert np.allclose(o[0, h], orc.rope(rf[0], R, THETA, -1), atol=1e-12)
    # window 0 and one selected entry: output = RoPE^-1(p) of that entry
    _, _, o, _ = orc.hybrid_attn(comp, raw, bt, [0], [400], q, topk=np.array([[17, -1]], np.int32), swa_window=0)
    assert np.allclose(o[0, 1], orc.rope(cf[17], R, THETA, -400), atol=1e-12)


def test_empty_key_set_is_zero(orc):
    comp, raw, bt, _, _ = make_layer(orc, 13, 256, 128, 32, 128)
    _, _, o, f = orc.hybrid_attn(comp, raw, bt, [0], [0], randn_bf16(13, 40, (1, 4, 128)), swa_window=128)
    assert f == 0 and np.all(o == 0)


def test_c128a_early_queries_are_plain_window_attention(orc):
    T, D, R, S = 512, 128, 32, 128
    comp, raw, bt, cf, rf = make_layer(orc, 14, T, D, R, 128)
    pos = np.array([5, 64, 127], np.int64)
    q = randn_bf16(14, 40, (3, 4, D))
    qf = bf16_to_f64(q)
    _, _, o, _ = orc.hybrid_attn(comp, raw, bt, np.zeros(3, np.int32), pos, q, swa_window=S)
    for n, p in enumerate(pos):
        K = rf[max(0, p - S):p]
        z = qf[n] @ K.T / np.sqrt(D)
        a = np.exp(z - z.max(1, keepdims=True))
        a /= a.sum(1, keepdims=True)
        for h in range(4):
            assert np.allclose(o[n, h], orc.rope(a[h] @ K, R, THETA, -int(p)), atol=1e-12)


def test_topk_covering_all_equals_dense(orc):
    T, D, R = 1024, 128, 32
    comp, raw, bt, _, _ = make_layer(orc, 15, T, D, R, 4)
    pos = np.array([200, 1024], np.int64)
    q = randn_bf16(15, 40, (2, 8, D))
    k = 256
    topk = np.full((2, k), -1, np.int32)
    for n, p in enumerate(pos):
        topk[n, :p // 4] = np.arange(p // 4)
    _, _, a, _ = orc.hybrid_attn(comp, raw, bt, [0, 0], pos, q, topk=topk)
    _, _, b, _ = orc.hybrid_attn(comp, raw, bt, [0, 0], pos, q, topk=None)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-13)


def test_shift_invariance(orc):
    """Moving every key and the query by delta positions (q re-rotated) leaves the
    output unchanged: the purpose of the inverse RoPE ([Notes] Inverse RoPE 的数学原理).
    fp32 rows; q is bf16, so the two queries differ by bf16 rounding only."""
    D, R, S, H = 128, 32, 64, 4
    base_p = 600
    rs = np.random.default_rng(8)
    cvals = rs.standard_normal((base_p // 4, D))
    rvals = rs.standard_normal((base_p, D))
    q0 = rs.standard_normal((H, D))
    outs = []
    for delta in [0, 128 * 5, 1 << 20]:
        T = base_p + delta
        mb = T // 256 + 1
        bt = np.full((1, mb), -1, np.int32)          # only the blocks in use are mapped
        used = sorted({(delta + t) // 256 for t in range(base_p)})
        bt[0, used] = np.arange(len(used))
        comp = orc.HostPool(4, 1, D, R, THETA, orc.F32, len(used), state=False)
        raw = orc.HostPool(1, 1, D, R, THETA, orc.F32, len(used), state=False)
        for i in range(base_p // 4):
            si = i + delta // 4
            pg, r = bt[0, (4 * si) // 256], si % 64
            comp.rows[pg, r] = orc.rope(cvals[i], R, THETA, 4 * si).astype(np.float32).view(np.uint8)
        for t in range(base_p - S, base_p):
            tt = t + delta
            raw.rows[bt[0, tt // 256], tt % 256] = orc.rope(rvals[t], R, THETA, tt).astype(np.float32).view(np.uint8)
        qr = np.stack([orc.rope(q0[h], R, THETA, base_p + delta) for h in range(H)])
        qb = (qr.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        topk = (np.array([[3, 50, 99, 149]]) + delta // 4).astype(np.int32)
        _, _, o, f = orc.hybrid_attn(comp, raw, bt, [0], [base_p + delta], qb[None], topk=topk, swa_window=S)
        assert f == 0
        outs.append(o)
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) < 1e-2


def test_fp8_kv_and_output(orc):
    T, D, R, H = 512, 128, 32, 4
    comp, raw, bt, cf, rf = make_layer(orc, 16, T, D, R, 4, kv_dtype=orc.FP8)
    pos = np.array([300, 512], np.int64)
    q = randn_bf16(16, 40, (2, H, D))
    topk = np.array([[1, 5, 9, 70], [0, 2, 100, 127]], np.int32)
    out, sc, o64, f = orc.hybrid_attn(comp, raw, bt, [0, 0], pos, q, topk=topk, out_dtype=orc.FP8)
    assert f == 0
    want = twin(orc, bf16_to_f64(q), pos, cf, rf, 4, [set(t.tolist()) for t in topk], 128, R, D ** -0.5)
    assert np.allclose(o64, want, rtol=1e-12, atol=1e-12)
    g = o64.reshape(2, H, D // 64, 64)
    assert np.allclose(sc, np.abs(g).max(-1) / 448.0, rtol=1e-6)
    table = np.array([orc.e4m3_to_f64(c) for c in range(256)])
    deq = table[out].reshape(2, H, D // 64, 64) * sc[..., None]
    r = np.abs(g) / sc[..., None]
    ulp = np.where(r < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(r, 1e-30))) - 3))
    assert np.all(np.abs(deq - g) <= sc[..., None] * ulp / 2 * (1 + 1e-6))


def test_bf16_output_rounding(orc):
    comp, raw, bt, _, _ = make_layer(orc, 17, 512, 128, 32, 128)
    q = randn_bf16(17, 40, (2, 4, 128))
    out, _, o64, _ = orc.hybrid_attn(comp, raw, bt, [0, 0], [256, 512], q, out_dtype=orc.BF16)
    import torch
    want = torch.from_numpy(o64.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # fp64 -> bf16 directly may differ from fp64 -> fp32 -> bf16 only at exact fp32 ties
    assert np.mean(out == want) > 0.999


def test_invalid_ids_and_unmapped_pages(orc):
    comp, raw, bt, cf, rf = make_layer(orc, 18, 512, 128, 32, 4)
    q = randn_bf16(18, 40, (1, 2, 128))
    # id 100 is not visible at p = 300 (needs 4*101 <= 300): skipped and counted
    _, _, o, f = orc.hybrid_attn(comp, raw, bt, [0], [300], q, topk=np.array([[5, 100, -1]], np.int32))
    _, _, o2, f2 = orc.hybrid_attn(comp, raw, bt, [0], [300], q, topk=np.array([[5, -1, -1]], np.int32))
    assert f == 1 and f2 == 0 and np.array_equal(o, o2)
    bt2 = bt.copy()
    bt2[0, 0] = -1
    _, _, _, f3 = orc.hybrid_attn(comp, raw, bt2, [0], [300], q, topk=np.array([[5, 60, -1]], np.int32))
    assert f3 == 2 + (256 - 172)  # entries 5 and 60 (positions 20, 240: page 0) + raw tokens 172..255


def test_swa_only_layer(orc):
    _, raw, bt, _, rf = make_layer(orc, 19, 512, 128, 32, 4)
    q = randn_bf16(19, 40, (1, 2, 128))
    _, _, o, f = orc.hybrid_attn(None, raw, bt, [0], [300], q)
    want = twin(orc, bf16_to_f64(q), np.array([300]), np.zeros((0, 128)), rf, 4, None, 128, 32, 128 ** -0.5)
    assert f == 0 and np.allclose(o, want, atol=1e-12)

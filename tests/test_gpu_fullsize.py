"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (bench.DecodeSetup / bench.PrefillSetup issue the calls), on
sampled outputs that the oracle computes one by one:

  * c128a decode, 8 sequences x 32768 tokens (dense over 256 entries + window);
  * c4a decode, 16 x 131072 tokens, top-512 + window (the benchmarked step);
  * 1M-token hybrid decode, fp8 caches and fp8 output, both layer kinds;
  * c4a prefill, 8192 new tokens on a 65536-token prefix, fp8 output.

For each sampled query the oracle recomputes, from the seeded inputs alone,
the index top-k over every visible entry, the stored rows that query reads
(compressed entries from their token windows, raw window rows), and the
attention output; the GPU's rows, ids and outputs are checked against them.
Where the output is fp8 (one e4m3 ULP of the oracle's quantisation), the
GPU's rows are first checked against the oracle's, then the oracle's rows are
written into the GPU pools and only the attention call is re-run, so both
sides quantise an output computed from the same rows.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from synth import workloads as W
from tests.gpu_util import DEV, assert_close, assert_fp4_close, assert_fp8_close, assert_topk_equivalent, host, host_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csl():
    import compressed_sparse_long_amd as c
    return c


def say(msg):
    print(f"[fullsize] {msg}", flush=True)


def gpu_rows(pool, bt_row: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Stored rows of entries `ids` of one sequence, read from a GPU pool."""
    per = 256 // pool.ratio
    pages = torch.from_numpy(bt_row[(ids * pool.ratio) // 256].astype(np.int64)).to(DEV)
    slots = torch.from_numpy((ids % per).astype(np.int64)).to(DEV)
    return host(pool.rows[pages, slots])


def windows(x_seq: torch.Tensor, lg_seq: torch.Tensor | None, ids: np.ndarray, ratio: int, coff: int):
    """Window tokens r(i+1)-W .. r(i+1)-1 of each entry (negative positions
    clamped to 0: the oracle ignores them) from a sequence's inputs on the GPU."""
    Wn = coff * ratio
    t = ids[:, None].astype(np.int64) * ratio + ratio - Wn + np.arange(Wn)[None, :]
    ti = torch.from_numpy(np.clip(t, 0, None)).to(x_seq.device)
    xw = host_u16(x_seq[ti])
    lw = None if lg_seq is None else host(lg_seq[ti])
    return xw, lw


def oracle_rows(pool, ids, x_seq, lg_seq, gain, theta, chunk=1024):
    out = []
    for c0 in range(0, len(ids), chunk):
        sl = ids[c0:c0 + chunk]
        xw, lw = windows(x_seq, lg_seq, sl, pool.ratio, pool.coff)
        out.append(O.compress_rows(pool.ratio, pool.coff, pool.dim, pool.rope_dims, theta, pool.dtype, sl, xw, lw,
                                   None if gain is None else host(gain)))
    return np.concatenate(out)


def check_rows(got: np.ndarray, want: np.ndarray, dim: int, dtype: int, what: str):
    if dtype == O.FP8:
        sg = got[:, dim:].copy().view(np.float32)
        so = want[:, dim:].copy().view(np.float32)
        assert_fp8_close(O, got[:, :dim], sg, want[:, :dim], so, what=what)
    else:
        assert_close(O.decode_rows(got, dim, dtype), O.decode_rows(want, dim, dtype), what=what)


def put_rows(pool, bt_row: np.ndarray, ids: np.ndarray, rows: np.ndarray):
    """Write rows (the oracle's) into a GPU pool at entries `ids` of one sequence."""
    per = 256 // pool.ratio
    pages = torch.from_numpy(bt_row[(ids * pool.ratio) // 256].astype(np.int64)).to(DEV)
    slots = torch.from_numpy((ids % per).astype(np.int64)).to(DEV)
    pool.rows[pages, slots] = torch.from_numpy(np.ascontiguousarray(rows)).to(DEV)


def host_pool(ratio, coff, dim, rope_dims, theta, dtype, n_pages, ids, rows):
    """An oracle pool for one sequence (identity block table) holding `rows` at entries `ids`."""
    p = O.HostPool(ratio, coff, dim, rope_dims, theta, dtype, n_pages, state=False)
    per = 256 // ratio
    p.rows[(ids * ratio) // 256, ids % per] = rows
    return p


def check_out(csl, got_t, scales_t, o_out, o_scales, o64, dtype, what):
    if dtype == O.FP8:
        assert_fp8_close(O, host(got_t), host(scales_t), o_out, o_scales, what=what)
    elif dtype == O.BF16:
        assert_close(O.bf16_array_to_f64(host_u16(got_t)), o64, what=what)
    else:
        assert_close(host(got_t), o64, what=what)


def decode_query_check(csl, w, st, s, layer, theta=10000.0):
    """Oracle check of query s (one per sequence, at p = ctx) of a decode step
    already run by `st` (a bench.DecodeSetup, replica 0)."""
    T, D, R, DI = w.ctx, w.dim, w.rope_dims, w.idx_dim
    p = T
    mb = w.max_blocks
    bt_row = host(st.bt[s])
    rep = st.reps[0]
    x_seq = W.latent(w, s, 0, T + 1, device=DEV)
    raw_ids = np.arange(p - w.swa, p + 1)                       # the window, plus the token the step inserted
    raw_o = oracle_rows(rep["raw"], raw_ids, x_seq, None, None, theta)
    check_rows(gpu_rows(rep["raw"], bt_row, raw_ids), raw_o, D, w.kv_dtype, f"{layer} seq {s}: raw rows")
    raw_pool = host_pool(1, 1, D, R, theta, w.kv_dtype, mb, raw_ids[:-1], raw_o[:-1])
    bt_o = np.arange(mb, dtype=np.int32)[None]
    q = host_u16(st.q[s:s + 1])
    if layer == "c4a":
        nv = p // 4
        if w.synth_index_keys:
            keys = host_u16(W.index_keys(w, s, 0, nv, device=DEV))
            idx_pool = O.HostPool(4, 2, DI, 0, theta, O.BF16, mb, state=False)
            idx_pool.rows.reshape(-1, DI * 2)[:nv] = keys.view(np.uint8).reshape(nv, DI * 2)
        else:
            # index rows written by the compressor (fp4 here): every visible entry against
            # the oracle's compressor over the same latents; the top-k is then checked on
            # the GPU's own rows, so both sides score the same bytes
            idt = O.FP4 if w.idx_dtype == 3 else O.BF16
            xi = host_u16(W.latent(w, s, 0, T + 1, dim=DI, tid=W.T_XI, device=DEV))
            lgi = host(W.logits(w, s, 0, T + 1, 2, tid=W.T_LOGITS_I, device=DEV))
            o_idx = O.HostPool(4, 2, DI, 0, theta, idt, mb)
            gi = W.gain(w, DI, tid=W.T_GAIN_I, device=DEV)
            assert O.compress_insert(o_idx, bt_o, [0], [0, T + 1], xi, lgi, None if gi is None else host(gi)) == 0
            ents = np.arange(nv)
            g_rows = gpu_rows(rep["idx"], bt_row, ents)
            o_rows = o_idx.rows.reshape(-1, o_idx.row_bytes)[:nv]
            if idt == O.FP4:
                assert_fp4_close(O, g_rows, o_rows, DI, what=f"c4a seq {s}: fp4 index rows")
            else:
                check_rows(g_rows, o_rows, DI, idt, f"c4a seq {s}: index rows")
            idx_pool = O.HostPool(4, 2, DI, 0, theta, idt, mb, state=False)
            idx_pool.rows.reshape(-1, idx_pool.row_bytes)[:nv] = g_rows
        o_topk, o_kth, o_sc, _ = O.index_topk(idx_pool, bt_o, [0], [p], host_u16(st.q_idx[s:s + 1]),
                                              host(st.w_idx[s:s + 1]), w.topk, want_scores=True, max_cand=nv)
        g_topk = host(st.topk[s:s + 1])
        assert_topk_equivalent(g_topk, o_topk, o_sc, o_kth, what=f"c4a seq {s}")
        # the attention is checked over the GPU's ids (the oracle's up to allowed swaps)
        ids = g_topk[0][g_topk[0] >= 0].astype(np.int64)
        lg_seq = W.logits(w, s, 0, T + 1, 2, device=DEV)
        main_o = oracle_rows(rep["main4"], ids, x_seq, lg_seq, st.gain, theta)
        check_rows(gpu_rows(rep["main4"], bt_row, ids), main_o, D, w.kv_dtype, f"c4a seq {s}: top-k entries")
        comp = host_pool(4, 2, D, R, theta, w.kv_dtype, mb, ids, main_o)
        topk_arg = g_topk
        same = np.array_equal(g_topk, o_topk)
    else:
        ids = np.arange(p // 128, dtype=np.int64)
        lg_seq = W.logits(w, s, 0, T + 1, 1, tid=W.T_LOGITS_128, device=DEV)
        main_o = oracle_rows(rep["main128"], ids, x_seq, lg_seq, None, theta)
        check_rows(gpu_rows(rep["main128"], bt_row, ids), main_o, D, w.kv_dtype, f"c128a seq {s}: entries")
        comp = host_pool(128, 1, D, R, theta, w.kv_dtype, mb, ids, main_o)
        topk_arg = None
        same = True
    o_out, o_sc8, o64, f = O.hybrid_attn(comp, raw_pool, bt_o, [0], [p], q, topk=topk_arg, swa_window=w.swa,
                                         softmax_scale=st.scale, out_dtype=w.out_dtype)
    assert f == 0
    if w.out_dtype == O.FP8:
        # fp8 outputs are held to one e4m3 ULP of the oracle's quantisation; the
        # rows each side computed may differ by a code (checked above), so the
        # query's attention is re-run over the oracle's rows
        put_rows(rep["raw"], bt_row, raw_ids[:-1], raw_o[:-1])
        put_rows(rep["main4" if layer == "c4a" else "main128"], bt_row, ids, main_o)
        st.attend(0)
        torch.cuda.synchronize()
        assert csl.read_device_error() == 0
    sc = st.out_scales[layer]
    check_out(csl, st.out[layer][s:s + 1], None if sc is None else sc[s:s + 1], o_out, o_sc8, o64, w.out_dtype,
              f"{layer} seq {s}: attention output")
    return same


def run_decode(csl, w):
    from bench import DecodeSetup
    say(f"{w.name}: building caches")
    st = DecodeSetup(w, 1, fused_inserts=True)
    say(f"{w.name}: one decode step")
    st.step(0)
    torch.cuda.synchronize()
    assert csl.read_device_error() == 0
    return st


def test_c128a_decode_full_size(csl):
    w = W.c128a_decode()
    st = run_decode(csl, w)
    for s in (0, 3, 7):
        say(f"{w.name}: oracle check of sequence {s}")
        decode_query_check(csl, w, st, s, "c128a")
    del st
    torch.cuda.empty_cache()


def test_c4a_decode_full_size(csl):
    w = W.c4a_decode()
    st = run_decode(csl, w)
    for s in range(w.num_seqs):
        say(f"{w.name}: oracle check of sequence {s}")
        decode_query_check(csl, w, st, s, "c4a")
    del st
    torch.cuda.empty_cache()


def test_c4a_fp4_index_decode_full_size(csl):
    w = W.c4a_decode_fp4()
    st = run_decode(csl, w)
    for s in (0, 15):
        say(f"{w.name}: oracle check of sequence {s}")
        decode_query_check(csl, w, st, s, "c4a")
    del st
    torch.cuda.empty_cache()


def test_1m_hybrid_decode_full_size(csl):
    w = W.long_1m()
    st = run_decode(csl, w)
    say(f"{w.name}: oracle check, c4a layer")
    decode_query_check(csl, w, st, 0, "c4a")
    say(f"{w.name}: oracle check, c128a layer")
    decode_query_check(csl, w, st, 0, "c128a")
    del st
    torch.cuda.empty_cache()


PREFILL_SAMPLES = (0, 1, 3, 127, 128, 2049, 4095, 8190, 8191)


def test_c4a_prefill_full_size(csl):
    from bench import PrefillSetup
    w = W.prefill()
    theta = w.theta
    say(f"{w.name}: building the prefix")
    st = PrefillSetup(w)
    say(f"{w.name}: one prefill step")
    st.step()
    torch.cuda.synchronize()
    assert csl.read_device_error() == 0
    T0, n, D, R, DI = w.ctx, w.new_tokens, w.dim, w.rope_dims, w.idx_dim
    Tn = T0 + n
    mb = w.max_blocks
    bt_row = host(st.bt[0])
    bt_o = np.arange(mb, dtype=np.int32)[None]
    # index entries: the oracle's streaming insert over the whole sequence
    say(f"{w.name}: oracle index cache")
    xi = host_u16(W.latent(w, 0, 0, Tn, dim=DI, tid=W.T_XI, device=DEV))
    lgi = host(W.logits(w, 0, 0, Tn, 2, tid=W.T_LOGITS_I, device=DEV))
    idx_pool = O.HostPool(4, 2, DI, 0, theta, O.BF16, mb)
    assert O.compress_insert(idx_pool, bt_o, [0], [0, Tn], xi, lgi, host(st.gain_i)) == 0
    ent = np.concatenate([np.arange(0, 8), np.arange(T0 // 4 - 4, T0 // 4 + 4), np.arange(Tn // 4 - 8, Tn // 4)])
    check_rows(gpu_rows(st.idx, bt_row, ent), idx_pool.rows[ent // 64, ent % 64], DI, O.BF16, "prefill index rows")
    js = np.array(PREFILL_SAMPLES)
    jt = torch.from_numpy(js).to(DEV)
    pos = T0 + js
    q_seq = np.zeros(len(js), np.int32)
    o_topk, o_kth, o_sc, _ = O.index_topk(idx_pool, bt_o, q_seq, pos, host_u16(st.q_idx[jt]), host(st.w_idx[jt]),
                                          w.topk, want_scores=True, max_cand=int(pos.max()) // 4)
    g_topk = host(st.topk[jt])
    assert_topk_equivalent(g_topk, o_topk, o_sc, o_kth, what="prefill")
    # the rows the sampled queries read
    say(f"{w.name}: oracle rows of the sampled queries")
    x_seq = W.latent(w, 0, 0, Tn, device=DEV)
    lg_seq = W.logits(w, 0, 0, Tn, 2, device=DEV)
    # the attention is checked over the GPU's ids (the oracle's up to allowed swaps)
    ids = np.unique(g_topk[g_topk >= 0]).astype(np.int64)
    main_o = oracle_rows(st.main, ids, x_seq, lg_seq, st.gain, theta)
    check_rows(gpu_rows(st.main, bt_row, ids), main_o, D, w.kv_dtype, "prefill top-k entries")
    raw_ids = np.unique(np.concatenate([np.arange(max(0, p - w.swa), p) for p in pos])).astype(np.int64)
    raw_o = oracle_rows(st.raw, raw_ids, x_seq, None, None, theta)
    check_rows(gpu_rows(st.raw, bt_row, raw_ids), raw_o, D, w.kv_dtype, "prefill raw rows")
    comp = host_pool(4, 2, D, R, theta, w.kv_dtype, mb, ids, main_o)
    raw_pool = host_pool(1, 1, D, R, theta, w.kv_dtype, mb, raw_ids, raw_o)
    say(f"{w.name}: oracle attention of {len(js)} queries")
    o_out, o_sc8, o64, f = O.hybrid_attn(comp, raw_pool, bt_o, q_seq, pos, host_u16(st.q[jt]), topk=g_topk,
                                         swa_window=w.swa, softmax_scale=st.scale, out_dtype=w.out_dtype)
    assert f == 0
    # fp8 outputs: the sampled queries' attention re-run over the oracle's rows
    # (the rows themselves were compared above)
    put_rows(st.main, bt_row, ids, main_o)
    put_rows(st.raw, bt_row, raw_ids, raw_o)
    st.attend()
    torch.cuda.synchronize()
    assert csl.read_device_error() == 0
    check_out(csl, st.out[jt], st.out_scales[jt], o_out, o_sc8, o64, w.out_dtype, "prefill attention output")
    del st
    torch.cuda.empty_cache()

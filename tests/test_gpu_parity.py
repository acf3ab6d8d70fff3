"""GPU parity: every C-ABI call against the CPU oracle on the same seeded inputs.

Sizes span several tiles and ragged tails; tolerances are those of the method's acceptance rules:
rows and outputs rtol 1e-2 / atol 1e-2, fp8 within one e4m3 ULP of the
oracle's quantisation, top-k sets equal up to swaps within 1e-4 of the k-th
score.  Every case prints its name before its GPU step.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle as O
from tests.gpu_util import (DEV, assert_close, assert_fp4_close, assert_fp8_close, assert_topk_equivalent, dev,
                            dev_bf16, host, host_u16)
from tests.util import (bf16_to_f64, block_table, fp4_rows, gather_rows, rand_u, randn_bf16, randn_f32,
                        scatter_rows)

pytestmark = pytest.mark.gpu
THETA = 10000.0


@pytest.fixture(scope="module")
def csl():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import compressed_sparse_long_amd as m
    m.read_device_error()  # clear
    return m


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def gpu_pool(csl, hp: O.HostPool, state=True):
    """Device pool with the same bytes as a host pool."""
    p = csl.Pool(hp.ratio, hp.coff, hp.dim, hp.rope_dims, hp.theta, hp.dtype, hp.num_pages,
                 rows=dev(hp.rows), state=False)
    if state and hp.state_x is not None:
        p.state_x = dev(hp.state_x.view(np.int16), torch.bfloat16)
        p.state_logits = dev(hp.state_logits)
    return p


# ---------------------------------------------------------------------------
# compress_insert
# ---------------------------------------------------------------------------

COMPRESS_CASES = [
    dict(name="c4a_d128_r32_bf16_1seq", ratio=4, coff=2, D=128, R=32, dtype=O.BF16, lens=[1024],
         chunks=[[1024]]),
    dict(name="c4a_d512_r64_fp8_2seq_ragged_chunks", ratio=4, coff=2, D=512, R=64, dtype=O.FP8, lens=[700, 413],
         chunks=[[300, 1, 399], [5, 0, 408]]),
    dict(name="c128a_d512_r64_bf16_3seq_chunked", ratio=128, coff=1, D=512, R=64, dtype=O.BF16,
         lens=[1100, 640, 129], chunks=[[127, 500, 473], [640, 0, 0], [1, 127, 1]]),
    dict(name="c128a_d512_fp8", ratio=128, coff=1, D=512, R=64, dtype=O.FP8, lens=[768], chunks=[[700, 68]]),
    dict(name="raw_d512_bf16_2seq", ratio=1, coff=1, D=512, R=64, dtype=O.BF16, lens=[300, 77], chunks=[[200, 100],
                                                                                                         [77, 0]]),
    dict(name="raw_d512_fp8", ratio=1, coff=1, D=512, R=64, dtype=O.FP8, lens=[260], chunks=[[260]]),
    dict(name="index_d32_norope", ratio=4, coff=2, D=32, R=0, dtype=O.BF16, lens=[1024], chunks=[[1000, 24]]),
    dict(name="index_d128_gain", ratio=4, coff=2, D=128, R=0, dtype=O.BF16, lens=[520], chunks=[[3, 517]],
         gain=True),
    dict(name="c4a_d512_gain_start_offset", ratio=4, coff=2, D=512, R=64, dtype=O.BF16, lens=[600],
         chunks=[[0, 600]], gain=True),
    # fp4 (MXFP4) index rows, ragged chunks over two sequences
    dict(name="index_d128_fp4", ratio=4, coff=2, D=128, R=0, dtype=O.FP4, lens=[1100, 300],
         chunks=[[600, 1, 499], [300]], gain=True),
]


@pytest.mark.parametrize("case", COMPRESS_CASES, ids=[c["name"] for c in COMPRESS_CASES])
def test_compress_insert_parity(csl, orc, case):
    r, c, D, R, dt = case["ratio"], case["coff"], case["D"], case["R"], case["dtype"]
    lens, chunks = case["lens"], case["chunks"]
    ns = len(lens)
    seed = zlib.crc32(case["name"].encode()) % 1000
    mb = max(lens) // 256 + 1
    bt = block_table(seed, ns, mb, extra_pages=2)
    npages = ns * mb + 2
    hp = O.HostPool(r, c, D, R, THETA, dt, npages)
    gp = gpu_pool(csl, hp)
    gbt = dev(bt)
    xs = [randn_bf16(seed, 100 + s, (lens[s], D)) for s in range(ns)]
    ls = [randn_f32(seed, 200 + s, (lens[s], c)).astype(np.float32) for s in range(ns)]
    gain = rand_u(seed, 300, (D,), 0.5, 1.5).astype(np.float32) if case.get("gain") else None
    done = [0] * ns
    for rnd in range(max(len(ch) for ch in chunks)):
        sizes = [chunks[s][rnd] if rnd < len(chunks[s]) else 0 for s in range(ns)]
        cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        st = np.array(done, np.int64)
        x = np.concatenate([xs[s][done[s]:done[s] + sizes[s]] for s in range(ns)])
        lg = np.concatenate([ls[s][done[s]:done[s] + sizes[s]] for s in range(ns)]) if r > 1 else None
        assert O.compress_insert(hp, bt, st, cu, x, lg, gain) == 0
        say(f"compress {case['name']} round {rnd} sizes {sizes}")
        csl.compress_insert(gp, gbt, dev(st), dev(cu), dev_bf16(x), None if lg is None else dev(lg),
                            None if gain is None else dev(gain))
        done = [done[s] + sizes[s] for s in range(ns)]
    torch.cuda.synchronize()
    assert csl.read_device_error() == 0
    g_rows = host(gp.rows)
    for s in range(ns):
        n_ent = lens[s] // r
        go = gather_rows(g_rows, bt, s, r, 0, n_ent)
        oo = gather_rows(hp.rows, bt, s, r, 0, n_ent)
        if dt == O.BF16:
            assert_close(O.decode_rows(go, D, dt), O.decode_rows(oo, D, dt), what=f"{case['name']} seq {s}")
        elif dt == O.FP4:
            assert_fp4_close(O, go, oo, D, what=f"{case['name']} seq {s}")
        else:
            assert_fp8_close(orc, go[:, :D], go[:, D:].copy().view(np.float32), oo[:, :D],
                             oo[:, D:].copy().view(np.float32), what=f"{case['name']} seq {s}")
    if r > 1:
        assert np.array_equal(host_u16(gp.state_x), hp.state_x)
        assert np.array_equal(host(gp.state_logits), hp.state_logits)


def test_compress_insert_multi_parity(csl, orc):
    """Raw window, c4a main (fp8) and c4a index pools filled by one fused launch per
    chunk, against the oracle's one-pool inserts."""
    seed, D, DI, R = 17, 512, 128, 64
    lens, chunks = [600, 333], [[250, 1, 349], [333, 0, 0]]
    ns = len(lens)
    mb = max(lens) // 256 + 1
    bt = block_table(seed, ns, mb, extra_pages=1)
    P = ns * mb + 1
    hps = [O.HostPool(1, 1, D, R, THETA, O.BF16, P), O.HostPool(4, 2, D, R, THETA, O.FP8, P),
           O.HostPool(4, 2, DI, 0, THETA, O.BF16, P)]
    gps = [gpu_pool(csl, h) for h in hps]
    xs = [randn_bf16(seed, 100 + s, (lens[s], D)) for s in range(ns)]
    xis = [randn_bf16(seed, 110 + s, (lens[s], DI)) for s in range(ns)]
    ls = [randn_f32(seed, 200 + s, (lens[s], 2)).astype(np.float32) for s in range(ns)]
    lis = [randn_f32(seed, 210 + s, (lens[s], 2)).astype(np.float32) for s in range(ns)]
    gain = rand_u(seed, 300, (D,), 0.5, 1.5).astype(np.float32)
    done = [0] * ns
    for rnd in range(3):
        sizes = [chunks[s][rnd] for s in range(ns)]
        cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        st = np.array(done, np.int64)
        cat = lambda arrs: np.concatenate([arrs[s][done[s]:done[s] + sizes[s]] for s in range(ns)])
        x, xi, lg, li = cat(xs), cat(xis), cat(ls), cat(lis)
        assert O.compress_insert(hps[0], bt, st, cu, x) == 0
        assert O.compress_insert(hps[1], bt, st, cu, x, lg, gain) == 0
        assert O.compress_insert(hps[2], bt, st, cu, xi, li) == 0
        say(f"compress_insert_multi round {rnd} sizes {sizes}")
        csl.compress_insert_multi([(gps[0], dev_bf16(x), None, None), (gps[1], dev_bf16(x), dev(lg), dev(gain)),
                                   (gps[2], dev_bf16(xi), dev(li), None)], dev(bt), dev(st), dev(cu))
        done = [done[s] + sizes[s] for s in range(ns)]
    torch.cuda.synchronize()
    assert csl.read_device_error() == 0
    for (h, g, r, what) in ((hps[0], gps[0], 1, "raw"), (hps[1], gps[1], 4, "main fp8"), (hps[2], gps[2], 4, "index")):
        for s in range(ns):
            go = gather_rows(host(g.rows), bt, s, r, 0, lens[s] // r)
            oo = gather_rows(h.rows, bt, s, r, 0, lens[s] // r)
            if h.dtype == O.BF16:
                assert_close(O.decode_rows(go, h.dim, h.dtype), O.decode_rows(oo, h.dim, h.dtype), what=what)
            else:
                assert_fp8_close(orc, go[:, :h.dim], go[:, h.dim:].copy().view(np.float32), oo[:, :h.dim],
                                 oo[:, h.dim:].copy().view(np.float32), what=what)


# ---------------------------------------------------------------------------
# q_norm_rope_insert (query side + raw-key insert)
# ---------------------------------------------------------------------------

# Launch forms by rows (tokens x (heads + 1)): one row per wave below 4096, two
# below 16384, four from there on; the cases below cover all three.
QSIDE_CASES = [
    dict(name="d512_r64_h64_bf16_2seq_chunked", D=512, R=64, H=64, dtype=O.BF16, lens=[300, 77],
         chunks=[[200, 100], [77, 0]], gain=True),
    dict(name="d512_r64_h16_fp8_inplace", D=512, R=64, H=16, dtype=O.FP8, lens=[260], chunks=[[1, 259]],
         in_place=True),
    dict(name="d128_r32_h8_tiny", D=128, R=32, H=8, dtype=O.BF16, lens=[1024], chunks=[[1000, 24]]),
    # 7 heads: a wave's four rows cross token boundaries
    dict(name="d512_h7_rows_cross_tokens", D=512, R=64, H=7, dtype=O.BF16, lens=[33, 50], chunks=[[33], [50]],
         gain=True),
    dict(name="d64_r16_h1_3seq_one_empty", D=64, R=16, H=1, dtype=O.BF16, lens=[5, 0, 9], chunks=[[5], [0], [9]]),
    # 297 tokens x 65 rows: four rows per wave (the large-launch form), fp8 key rows, ragged tail
    dict(name="d512_h64_fp8_four_rows_per_wave", D=512, R=64, H=64, dtype=O.FP8, lens=[257, 40],
         chunks=[[257], [40]], gain=True),
    # positions near 2^20: the angles of the fastest pairs reach ~1e6 rad
    dict(name="d512_h64_pos_1m", D=512, R=64, H=64, dtype=O.BF16, lens=[40], chunks=[[40]], start=(1 << 20) - 17),
]


def sparse_table(seed, lens, start, extra=0):
    """Block table mapping only the blocks that positions start .. start+len-1 touch (others -1)."""
    mb = (start + max(lens)) // 256 + 1
    bt = np.full((len(lens), mb), -1, np.int32)
    nxt = 0
    for s, n in enumerate(lens):
        for b in range(start // 256, (start + n - 1) // 256 + 1 if n else start // 256):
            bt[s, b] = nxt
            nxt += 1
    perm = np.random.default_rng(seed).permutation(nxt + extra).astype(np.int32)
    bt[bt >= 0] = perm[bt[bt >= 0]]
    return bt, nxt + extra


@pytest.mark.parametrize("case", QSIDE_CASES, ids=[c["name"] for c in QSIDE_CASES])
def test_q_norm_rope_insert_parity(csl, orc, case):
    D, R, H, dt, lens, chunks = case["D"], case["R"], case["H"], case["dtype"], case["lens"], case["chunks"]
    ns, start = len(lens), case.get("start", 0)
    seed = zlib.crc32(case["name"].encode()) % 1000
    bt, npages = sparse_table(seed, lens, start, extra=1)
    hp = O.HostPool(1, 1, D, R, THETA, dt, npages, state=False)
    gp = gpu_pool(csl, hp, state=False)
    gbt = dev(bt)
    xs = [randn_bf16(seed, 100 + s, (lens[s], D)) for s in range(ns)]
    qs = [randn_bf16(seed, 150 + s, (lens[s], H, D)) for s in range(ns)]
    gain = rand_u(seed, 300, (D,), 0.5, 1.5).astype(np.float32) if case.get("gain") else None
    done = [0] * ns
    for rnd in range(max(len(ch) for ch in chunks)):
        sizes = [chunks[s][rnd] if rnd < len(chunks[s]) else 0 for s in range(ns)]
        cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        st = np.array(done, np.int64) + start
        x = np.concatenate([xs[s][done[s]:done[s] + sizes[s]] for s in range(ns)])
        q = np.concatenate([qs[s][done[s]:done[s] + sizes[s]] for s in range(ns)])
        want, f = O.q_norm_rope_insert(hp, bt, st, cu, x, q, gain)
        assert f == 0
        say(f"q_norm_rope_insert {case['name']} round {rnd} sizes {sizes}")
        gq = dev_bf16(q)
        out = None if case.get("in_place") else torch.empty_like(gq)
        got = csl.q_norm_rope_insert(gp, gbt, dev(st), dev(cu), dev_bf16(x), gq, None if gain is None else dev(gain),
                                     q_out=out)
        if case.get("in_place"):
            assert got is gq
        torch.cuda.synchronize()
        gotq = host_u16(got).reshape(want.shape)
        assert_close(bf16_to_f64(gotq), bf16_to_f64(want), what=f"{case['name']} q round {rnd}")
        if want.size:
            assert np.mean(gotq == want) >= 0.99, f"{case['name']}: {np.mean(gotq == want):.4f} bit-exact"
        done = [done[s] + sizes[s] for s in range(ns)]
    assert csl.read_device_error() == 0
    g_rows = host(gp.rows)
    for s in range(ns):
        go = gather_rows(g_rows, bt, s, 1, start, lens[s])
        oo = gather_rows(hp.rows, bt, s, 1, start, lens[s])
        if dt == O.BF16:
            assert_close(O.decode_rows(go, D, dt), O.decode_rows(oo, D, dt), what=f"{case['name']} rows seq {s}")
        else:
            assert_fp8_close(orc, go[:, :D], go[:, D:].copy().view(np.float32), oo[:, :D],
                             oo[:, D:].copy().view(np.float32), what=f"{case['name']} rows seq {s}")


def test_q_side_unmapped_page_flags_and_writes_queries(csl, orc):
    D, R, H = 512, 64, 4
    bt = np.array([[0, -1]], np.int32)
    hp = O.HostPool(1, 1, D, R, THETA, O.BF16, 2, state=False)
    gp = gpu_pool(csl, hp, state=False)
    x = randn_bf16(5, 1, (3, D))
    q = randn_bf16(5, 2, (3, H, D))
    st, cu = np.array([254], np.int64), np.array([0, 3], np.int32)
    want, f = O.q_norm_rope_insert(hp, bt, st, cu, x, q)
    assert f == 1
    say("q_norm_rope_insert unmapped page")
    got = csl.q_norm_rope_insert(gp, dev(bt), dev(st), dev(cu), dev_bf16(x), dev_bf16(q), q_out=torch.empty(
        (3, H, D), dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert csl.read_device_error() == csl.DEVERR_UNMAPPED_PAGE
    assert_close(bf16_to_f64(host_u16(got).reshape(want.shape)), bf16_to_f64(want), what="q")
    assert np.array_equal(host(gp.rows), hp.rows)


# ---------------------------------------------------------------------------
# index_topk
# ---------------------------------------------------------------------------

INDEX_CASES = [
    dict(name="h4_d32_k64", H=4, DI=32, k=64, pos=[[0, 3, 4, 7, 255, 256, 257, 259, 260, 1023, 1024]]),
    dict(name="h16_d128_k512_2seq", H=16, DI=128, k=512, pos=[[2047, 2048, 2051, 9000, 20000], [4, 5000, 6000]]),
    dict(name="h16_d64_k100", H=16, DI=64, k=100, pos=[[401, 403, 404, 3000, 3003]]),
    dict(name="h13_d128_k2048", H=13, DI=128, k=2048, pos=[[8191, 8192, 12000, 40000]]),
    # every score equal: the k-th score is shared by all candidates, ties go to the lower ids
    dict(name="h4_d32_k64_all_ties", H=4, DI=32, k=64, pos=[[1000, 1024]], mode="equal"),
    # a few huge scores far above the rest: fewer than k keys near the maximum
    dict(name="h16_d128_k512_outliers", H=16, DI=128, k=512, pos=[[20000, 131072]], mode="outlier"),
    # more than 32768 candidates: the select reads its keys from global memory
    dict(name="h16_d128_k512_40k_candidates", H=16, DI=128, k=512, pos=[[160000, 150003]]),
    # 400 000 visible entries: 392 chunks x 16 candidates, the 1024-thread merge
    dict(name="h16_d128_k512_merge_1024_threads", H=16, DI=128, k=512, pos=[[1600003]]),
    # scores rise with the id (with bf16 ties): the top 512 crowd the last chunks, so the
    # two-stage select's check fails and the exact single-pass select takes over
    dict(name="h16_d128_k512_ramp", H=16, DI=128, k=512, pos=[[131072, 70001]], mode="ramp"),
    # 64+ queries: the query-blocked score kernel.  A prefill-like run of 100
    # consecutive positions (6 full 16-query blocks and a ragged one)
    dict(name="tiled_h16_d128_k512_prefill", H=16, DI=128, k=512, pos=[list(range(9000, 9100))]),
    # three sequences, queries shuffled so every 16-query block mixes sequences,
    # positions from 0 (nothing visible) past k entries, chunk-ragged
    dict(name="tiled_h4_d32_k64_mixed", H=4, DI=32, k=64,
         pos=[[0, 3, 4, 5, 255, 256, 300] + list(range(4096, 4121)), list(range(1020, 1050)),
              [260 + 37 * i for i in range(20)]], shuffle=True),
    dict(name="tiled_h16_d64_k100_ties", H=16, DI=64, k=100, pos=[list(range(6000, 6070))], mode="equal"),
    # scores rise with the id: the top 512 crowd the last chunk, so after the
    # query-blocked scores and the stand-alone first stage the merge's candidate
    # check fails and its exact select over the score rows takes over
    dict(name="tiled_h16_d128_k512_ramp_fallback", H=16, DI=128, k=512, pos=[list(range(20000, 20070))],
         mode="ramp"),
    # fp4 (MXFP4) index rows: one query per score row, and query-blocked
    dict(name="fp4_h16_d128_k512_2seq", H=16, DI=128, k=512, pos=[[2047, 2048, 2051, 9000, 20000], [4, 5000, 6000]],
         fp4=True),
    dict(name="fp4_h16_d128_k512_outliers", H=16, DI=128, k=512, pos=[[20000, 131072]], mode="outlier", fp4=True),
    dict(name="tiled_fp4_h16_d128_k512_prefill", H=16, DI=128, k=512, pos=[list(range(9000, 9100))], fp4=True),
]


@pytest.mark.parametrize("case", INDEX_CASES, ids=[c["name"] for c in INDEX_CASES])
def test_index_topk_parity(csl, orc, case):
    H, DI, k = case["H"], case["DI"], case["k"]
    seed = zlib.crc32(case["name"].encode()) % 1000
    ns = len(case["pos"])
    max_pos = max(max(p) for p in case["pos"])
    mb = max_pos // 256 + 1
    bt = block_table(seed, ns, mb, extra_pages=1)
    fp4 = bool(case.get("fp4"))
    hp = O.HostPool(4, 2, DI, 0, THETA, O.FP4 if fp4 else O.BF16, ns * mb + 1, state=False)
    for s in range(ns):
        keys = randn_bf16(seed, 10 + s, (64 * mb, DI))
        if case.get("mode") == "equal":
            keys[:] = keys[0]
        elif case.get("mode") == "ramp":
            ramp = (1.0 + np.arange(64 * mb) / 8192.0).astype(np.float32)
            keys = (np.repeat(ramp[:, None], DI, 1).view(np.uint32) >> 16).astype(np.uint16)
        elif case.get("mode") == "outlier":
            keys = (keys.astype(np.uint32) - (12 << 7)).astype(np.uint16)       # x 2^-12 (exact in bf16)
            big = np.arange(7, 64 * mb, 997)                                      # ~1 in 1000 keeps its scale
            keys[big] = randn_bf16(seed, 30 + s, (len(big), DI))
        rows = fp4_rows(O, bf16_to_f64(keys)) if fp4 else keys.view(np.uint8).reshape(64 * mb, -1)
        scatter_rows(hp.rows, bt, s, 4, rows)
    q_seq = np.concatenate([[s] * len(p) for s, p in enumerate(case["pos"])]).astype(np.int32)
    q_pos = np.concatenate(case["pos"]).astype(np.int64)
    if case.get("shuffle"):
        perm = np.random.default_rng(seed).permutation(len(q_pos))
        q_seq, q_pos = q_seq[perm], q_pos[perm]
    nq = len(q_pos)
    qi = randn_bf16(seed, 20, (nq, H, DI))
    if case.get("mode") == "ramp":
        qi = (np.abs(O.bf16_array_to_f64(qi)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w = rand_u(seed, 21, (nq, H)).astype(np.float32)
    o_topk, o_kth, o_sc, f = O.index_topk(hp, bt, q_seq, q_pos, qi, w, k, want_scores=True, max_cand=max_pos // 4)
    assert f == 0
    gp = gpu_pool(csl, hp, state=False)
    topk = torch.full((nq, k), -7, dtype=torch.int32, device=DEV)
    kth = torch.empty(nq, dtype=torch.float32, device=DEV)
    ws = torch.empty(csl.index_topk_workspace(nq, max_pos, k) // 4, dtype=torch.float32, device=DEV)
    say(f"index_topk {case['name']} nq {nq} max_pos {max_pos}")
    csl.index_topk(gp, dev(bt), dev(q_seq), dev(q_pos), max_pos, dev_bf16(qi), dev(w), k, topk, kth, ws)
    torch.cuda.synchronize()
    assert csl.read_device_error() == 0
    assert_topk_equivalent(host(topk), o_topk, o_sc, o_kth, what=case["name"])
    g_kth = host(kth).astype(np.float64)
    for n in range(nq):
        if np.isneginf(o_kth[n]):
            assert np.isneginf(g_kth[n]) or g_kth[n] == np.inf
        else:
            assert abs(g_kth[n] - o_kth[n]) <= 1e-4 * max(1.0, abs(o_kth[n])) + 1e-6


# ---------------------------------------------------------------------------
# index_topk_insert: the indexer with the step's inserts in its top-k launch
# ---------------------------------------------------------------------------

FUSED_CASES = [
    # decode: one new token per sequence at the query's position; the index pool is
    # also an insert target (token 9003 closes entry 2250, not visible at p = 9003)
    dict(name="decode_two_stage_merge", pos=[[9003], [20000]], k=512),
    # short rows: a one-pass select, the inserts in a launch of their own
    dict(name="decode_short_rows", pos=[[1000], [700]], k=512),
    # 100 queries: the query-blocked scores, then the merge with 100 x 3 inserts
    dict(name="tiled_100_queries", pos=[list(range(9000, 9100))], k=512),
    # 150 000 visible entries: 148 chunks x 24 candidates, the 512-thread merge
    # (the inserts' workgroups run with their first 256 threads)
    dict(name="decode_wide_merge", pos=[[600003]], k=512, D=64, main_dtype=O.BF16, R=32),
    # the query side in the same launch (it owns the raw-window insert)
    dict(name="decode_with_query_side", pos=[[9003], [20000]], k=512, qside=True),
    dict(name="short_rows_with_query_side", pos=[[1000], [700]], k=512, qside=True),
    dict(name="wide_merge_with_query_side", pos=[[600003]], k=512, D=64, main_dtype=O.BF16, R=32, qside=True),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=[c["name"] for c in FUSED_CASES])
def test_index_topk_insert_equals_separate_calls(csl, orc, case):
    seed = zlib.crc32(case["name"].encode()) % 1000
    H, DI, D, R, k = 16, 128, case.get("D", 512), case.get("R", 64), case["k"]
    ns = len(case["pos"])
    max_pos = max(max(p) for p in case["pos"])
    mb = (max_pos + 256) // 256 + 1
    bt = block_table(seed, ns, mb, extra_pages=1)
    P = ns * mb + 1
    idx = O.HostPool(4, 2, DI, 0, THETA, O.BF16, P)
    for s in range(ns):
        scatter_rows(idx.rows, bt, s, 4, randn_bf16(seed, 10 + s, (64 * mb, DI)).view(np.uint8).reshape(64 * mb, -1))
    idx.state_x[:] = randn_bf16(seed, 11, idx.state_x.shape)
    idx.state_logits[:] = randn_f32(seed, 12, idx.state_logits.shape).astype(np.float32)
    raw = O.HostPool(1, 1, D, R, THETA, O.BF16, P, state=False)
    main = O.HostPool(4, 2, D, R, THETA, case.get("main_dtype", O.FP8), P)
    main.state_x[:] = randn_bf16(seed, 13, main.state_x.shape)
    main.state_logits[:] = randn_f32(seed, 14, main.state_logits.shape).astype(np.float32)
    q_seq = np.concatenate([[s] * len(p) for s, p in enumerate(case["pos"])]).astype(np.int32)
    q_pos = np.concatenate(case["pos"]).astype(np.int64)
    nq = len(q_pos)
    qi = randn_bf16(seed, 20, (nq, H, DI))
    w = rand_u(seed, 21, (nq, H)).astype(np.float32)
    # the new tokens: each sequence's queries' positions, in order
    lens = [len(p) for p in case["pos"]]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    st = np.array([p[0] for p in case["pos"]], np.int64)
    x = randn_bf16(seed, 30, (nq, D))
    xi = randn_bf16(seed, 31, (nq, DI))
    lg = randn_f32(seed, 32, (nq, 2)).astype(np.float32)
    li = randn_f32(seed, 33, (nq, 2)).astype(np.float32)
    gain = rand_u(seed, 34, (D,), 0.5, 1.5).astype(np.float32)
    qs = case.get("qside", False)
    qh = randn_bf16(seed, 35, (nq, 8, D))
    qg = rand_u(seed, 36, (D,), 0.5, 1.5).astype(np.float32)
    outs = []
    for fused in (False, True):
        gi, gr, gm = gpu_pool(csl, idx), gpu_pool(csl, raw, state=False), gpu_pool(csl, main)
        topk = torch.full((nq, k), -7, dtype=torch.int32, device=DEV)
        kth = torch.empty(nq, dtype=torch.float32, device=DEV)
        ws = torch.empty(csl.index_topk_workspace(nq, max_pos, k) // 4, dtype=torch.float32, device=DEV)
        jobs = [(gr, dev_bf16(x), None, None), (gm, dev_bf16(x), dev(lg), dev(gain)), (gi, dev_bf16(xi), dev(li), None)]
        gbt, gq, gw = dev(bt), dev_bf16(qi), dev(w)
        gqh, gqo = dev_bf16(qh), torch.empty((nq, 8, D), dtype=torch.bfloat16, device=DEV)
        qside = (gr, dev_bf16(x), gqh, dev(qg), gqo) if qs else None
        if qs:
            jobs = jobs[1:]  # the query side writes the raw rows
        say(f"index_topk_insert {case['name']} fused={fused}")
        if fused:
            csl.index_topk_insert(gi, gbt, dev(q_seq), dev(q_pos), max_pos, gq, gw, k, topk, jobs, dev(st), dev(cu),
                                  kth, ws, qside=qside)
        else:
            csl.index_topk(gi, gbt, dev(q_seq), dev(q_pos), max_pos, gq, gw, k, topk, kth, ws)
            csl.compress_insert_multi(jobs, gbt, dev(st), dev(cu))
            if qs:
                csl.q_norm_rope_insert(gr, gbt, dev(st), dev(cu), qside[1], gqh, qside[3], q_out=gqo)
        torch.cuda.synchronize()
        assert csl.read_device_error() == 0
        outs.append([host(topk), host(kth), host(gi.rows), host_u16(gi.state_x), host(gi.state_logits), host(gr.rows),
                     host(gm.rows), host_u16(gm.state_x), host(gm.state_logits), host_u16(gqo)])
    names = ["topk", "kth", "index rows", "index state_x", "index state_logits", "raw rows", "main rows",
             "main state_x", "main state_logits", "q_out"]
    for nm, a, b in zip(names, outs[0], outs[1]):
        if nm == "q_out" and not qs:
            continue
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{case['name']}: {nm} differ"
    # and the selection against the oracle on the pre-insert index pool
    o_topk, o_kth, o_sc, f = O.index_topk(idx, bt, q_seq, q_pos, qi, w, k, want_scores=True, max_cand=max_pos // 4)
    assert f == 0
    assert_topk_equivalent(outs[1][0], o_topk, o_sc, o_kth, what=case["name"])


# ---------------------------------------------------------------------------
# index_attn_decode: index scores + inserts, then merge + attention, two launches
# ---------------------------------------------------------------------------

def tail_table(seed, ns, mb, first_low, tail):
    """Block table in which blocks first_low[s] .. first_low[s] + tail - 1 of sequence s take
    pages [0, ns*tail) and every other block a page above them, so that a pool only read
    around the sequence's end (raw window, compressor state) can hold just the low pages
    (the others lie beyond its num_pages)."""
    lowp = np.random.default_rng(seed).permutation(ns * tail).astype(np.int32)
    highp = (ns * tail + np.random.default_rng(seed + 1).permutation(ns * (mb - tail))).astype(np.int32)
    bt = np.empty((ns, mb), np.int32)
    for s in range(ns):
        low = np.zeros(mb, bool)
        low[first_low[s]:first_low[s] + tail] = True
        bt[s, low] = lowp[s * tail:(s + 1) * tail]
        bt[s, ~low] = highp[s * (mb - tail):(s + 1) * (mb - tail)]
    return bt


FUSED_ATTN_CASES = [
    # two sequences, one query each: scores with first stage, inserts in the score launch,
    # the merge in the attention launch (8 candidates per thread)
    dict(name="two_stage_merge", pos=[[9003], [20000]]),
    # short rows (visible entries <= k): no first stage; the select kernel, then attention
    dict(name="short_rows", pos=[[1000], [700]]),
    # the query side (Q norm + RoPE, raw-key insert) in the score launch too
    dict(name="with_query_side", pos=[[9003], [20000]], qside=True),
    # 16 sequences (one query and one new token each), fp8 output: the precision variant
    dict(name="16_queries_fp8_out", pos=[[5000 + 700 * i] for i in range(16)], out=O.FP8),
    # index keys rising with the id: the top-k crowds the last chunk, the candidates'
    # check fails and every workgroup of the query takes the exact select on the score row
    dict(name="ramp_fallback", pos=[[9000], [12001]], mode="ramp", out=O.F32),
    # 150 000 visible entries: 148 chunks x 24 candidates, more than the attention launch
    # merges: the select launch runs between the two; no inserts; 48 heads (three head groups)
    dict(name="wide_candidates_select_launch", pos=[[600003]], DI=32, H=48, jobs=False),
    # fp8 keys (raw and c4a-main pools), with inserts into them, and fp8 output
    dict(name="fp8_keys_fp8_out", pos=[[9003], [20000], [14001]], kv=O.FP8, out=O.FP8),
]


@pytest.mark.parametrize("case", FUSED_ATTN_CASES, ids=[c["name"] for c in FUSED_ATTN_CASES])
def test_index_attn_decode_equals_separate_calls(csl, orc, case):
    seed = zlib.crc32(("fused_attn_" + case["name"]).encode()) % 1000
    HI, DI, D, R, k = 16, case.get("DI", 128), 512, 64, 512
    H = case.get("H", 64)
    od = case.get("out", O.BF16)
    ns = len(case["pos"])
    max_pos = max(max(p) for p in case["pos"])
    mb = (max_pos + 256) // 256 + 1
    # the window [p - 128, p - 1], the new token p and its entry's window [p - 7, p] lie in
    # blocks (p - 128) / 256 .. p / 256: three blocks from max(0, p / 256 - 1)
    tail = 3
    first_low = [max(0, max(p) // 256 - 1) for p in case["pos"]]
    bt = tail_table(seed, ns, mb, first_low, tail)
    P, P_low = ns * mb, ns * tail
    with_jobs = case.get("jobs", True)
    idx = O.HostPool(4, 2, DI, 0, THETA, O.BF16, P, state=with_jobs)
    for s in range(ns):
        keys = randn_bf16(seed, 10 + s, (64 * mb, DI))
        if case.get("mode") == "ramp":
            ramp = (1.0 + np.arange(64 * mb) / 8192.0).astype(np.float32)
            keys = (np.repeat(ramp[:, None], DI, 1).view(np.uint32) >> 16).astype(np.uint16)
        scatter_rows(idx.rows, bt, s, 4, keys.view(np.uint8).reshape(64 * mb, -1))
    kv = case.get("kv", O.BF16)

    def kv_rows(tid, n):
        if kv == O.FP8:
            return fp8_random_rows(seed, tid, n, D)
        return randn_bf16(seed, tid, (n, D)).view(np.uint8).reshape(n, -1)

    main = O.HostPool(4, 2, D, R, THETA, kv, P, state=with_jobs)
    for s in range(ns):
        scatter_rows(main.rows, bt, s, 4, kv_rows(40 + 2 * s, 64 * mb))
    raw = O.HostPool(1, 1, D, R, THETA, kv, P_low, state=False)
    for s in range(ns):
        n_raw = 256 * tail
        scatter_rows(raw.rows, bt, s, 1, kv_rows(100 + 2 * s, n_raw), i0=256 * first_low[s])
    if with_jobs:  # compressor state of the tail pages (the only pages the inserts read)
        for hp, t0 in ((idx, 11), (main, 13)):
            hp.state_x[:P_low] = randn_bf16(seed, t0, hp.state_x[:P_low].shape)
            hp.state_logits[:P_low] = randn_f32(seed, t0 + 1, hp.state_logits[:P_low].shape).astype(np.float32)
    q_seq = np.concatenate([[s] * len(p) for s, p in enumerate(case["pos"])]).astype(np.int32)
    q_pos = np.concatenate(case["pos"]).astype(np.int64)
    nq = len(q_pos)
    qi = randn_bf16(seed, 20, (nq, HI, DI))
    if case.get("mode") == "ramp":
        qi = (np.abs(O.bf16_array_to_f64(qi)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w = rand_u(seed, 21, (nq, HI)).astype(np.float32)
    q = randn_bf16(seed, 22, (nq, H, D))
    # new tokens: one per query, at the query's position (decode: the queries read below it)
    lens = [len(p) for p in case["pos"]]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    st = np.array([p[0] for p in case["pos"]], np.int64)
    x = randn_bf16(seed, 30, (nq, D))
    xi = randn_bf16(seed, 31, (nq, DI))
    lg = randn_f32(seed, 32, (nq, 2)).astype(np.float32)
    li = randn_f32(seed, 33, (nq, 2)).astype(np.float32)
    gain = rand_u(seed, 34, (D,), 0.5, 1.5).astype(np.float32)
    qs = case.get("qside", False)
    qh = randn_bf16(seed, 35, (nq, H, D))
    qg = rand_u(seed, 36, (D,), 0.5, 1.5).astype(np.float32)
    scale = D ** -0.5
    odt = {O.F32: torch.float32, O.BF16: torch.bfloat16, O.FP8: torch.uint8}[od]
    outs = []
    for fused in (False, True):
        gi, gr, gm = gpu_pool(csl, idx, state=with_jobs), gpu_pool(csl, raw, state=False), gpu_pool(csl, main, state=with_jobs)
        topk = torch.full((nq, k), -7, dtype=torch.int32, device=DEV)
        kth = torch.empty(nq, dtype=torch.float32, device=DEV)
        out = torch.empty((nq, H, D), dtype=odt, device=DEV)
        scales = torch.zeros((nq, H, D // 64), dtype=torch.float32, device=DEV) if od == O.FP8 else None
        jobs = []
        if with_jobs:
            jobs = [(gr, dev_bf16(x), None, None), (gm, dev_bf16(x), dev(lg), dev(gain)),
                    (gi, dev_bf16(xi), dev(li), None)]
        gbt, gq, gw = dev(bt), dev_bf16(qi), dev(w)
        gqh = dev_bf16(qh)
        gqo = gqh.clone() if qs else dev_bf16(q)
        qside = (gr, dev_bf16(x), gqh, dev(qg), gqo) if qs else None
        if qs:
            jobs = jobs[1:]  # the query side writes the raw rows
        say(f"index_attn_decode {case['name']} fused={fused} nq {nq}")
        if fused:
            ws = csl.workspace(csl.index_attn_decode_workspace(nq, H, max_pos, k, 128))
            csl.index_attn_decode(gi, gm, gr, gbt, dev(q_seq), dev(q_pos), max_pos, gq, gw, k, topk, gqo, 128, scale,
                                  od, out, scales, jobs, dev(st), dev(cu), kth, ws, qside=qside)
        else:
            wsi = torch.empty(csl.index_topk_workspace(nq, max_pos, k) // 4, dtype=torch.float32, device=DEV)
            wsa = csl.workspace(csl.hybrid_attn_workspace(nq, H, D, 4, k, 128, max_pos))
            if jobs or qs:
                csl.index_topk_insert(gi, gbt, dev(q_seq), dev(q_pos), max_pos, gq, gw, k, topk, jobs, dev(st),
                                      dev(cu), kth, wsi, qside=qside)
            else:
                csl.index_topk(gi, gbt, dev(q_seq), dev(q_pos), max_pos, gq, gw, k, topk, kth, wsi)
            csl.hybrid_attn_decode(gm, gr, gbt, dev(q_seq), dev(q_pos), max_pos, gqo, topk, k, 128, scale, od, out,
                                   scales, wsa)
        torch.cuda.synchronize()
        assert csl.read_device_error() == 0
        res = [host(topk), host(kth), host(out.view(torch.uint8)), host(gr.rows), host(gm.rows), host(gi.rows),
               host_u16(gqo)]
        if with_jobs:
            res += [host_u16(gm.state_x), host(gm.state_logits), host_u16(gi.state_x), host(gi.state_logits)]
        if od == O.FP8:
            res.append(host(scales))
        outs.append(res)
        if fused:  # the counter block is left zero
            assert not ws[:4096].any().item()
    names = ["topk", "kth", "out", "raw rows", "main rows", "index rows", "q", "main state_x", "main state_logits",
             "index state_x", "index state_logits", "out scales"]
    if not with_jobs:
        names = names[:7] + names[11:]
    for nm, a, b in zip(names, outs[0], outs[1]):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{case['name']}: {nm} differ"
    # against the oracle on the pre-insert pools: the selection, then the attention over the
    # GPU's ids for every query (the sets may differ from the oracle's by allowed swaps)
    o_topk, o_kth, o_sc, f = O.index_topk(idx, bt, q_seq, q_pos, qi, w, k, want_scores=True, max_cand=max_pos // 4)
    assert f == 0
    g_topk = outs[1][0]
    assert_topk_equivalent(g_topk, o_topk, o_sc, o_kth, what=case["name"])
    q_used = host_u16(gqo)
    o_out, o_oscale, o64, f = O.hybrid_attn(main, raw, bt, q_seq, q_pos, q_used, topk=g_topk, k=k, swa_window=128,
                                            softmax_scale=scale, out_dtype=od)
    assert f == 0
    g_out = outs[1][2]
    if od == O.F32:
        assert_close(g_out.view(np.float32).reshape(o64.shape), o64, what=case["name"])
    elif od == O.BF16:
        assert_close(O.bf16_array_to_f64(g_out.view(np.uint16).reshape(o64.shape)), o64, what=case["name"])
    else:
        assert_fp8_close(orc, g_out.reshape(o64.shape), outs[1][-1], o_out, o_oscale, what=case["name"])


# ---------------------------------------------------------------------------
# hybrid_attn_decode_insert: the step's inserts riding in the attention launch
# ---------------------------------------------------------------------------

DECODE_INSERT_CASES = [
    # the dense c128a step (every visible entry): raw and c128a-main inserts, one launch;
    # the third sequence's new token closes an entry (p + 1 a multiple of 128)
    dict(name="c128a_dense_bf16", ratio=128, coff=1, D=512, R=64, H=64, k=0, pos=[[9003], [20000], [12031]]),
    # fp8 keys and fp8 output
    dict(name="c128a_dense_fp8", ratio=128, coff=1, D=512, R=64, H=64, k=0, pos=[[9003], [16383]], kv=O.FP8,
         out=O.FP8),
    # c4a with given top-k ids (the index-free form of the step), 48 heads
    dict(name="c4a_given_ids", ratio=4, coff=2, D=512, R=64, H=48, k=512, pos=[[9003], [20000]]),
    # 128-dim keys: not the decode kernel; the inserts run first in a launch of their own
    dict(name="c4a_d128_inserts_first", ratio=4, coff=2, D=128, R=32, H=8, k=64, pos=[[3001], [1024]],
         out=O.F32),
]


@pytest.mark.parametrize("case", DECODE_INSERT_CASES, ids=[c["name"] for c in DECODE_INSERT_CASES])
def test_hybrid_attn_decode_insert_equals_separate_calls(csl, orc, case):
    seed = zlib.crc32(("decode_insert_" + case["name"]).encode()) % 1000
    D, R, H, k, r = case["D"], case["R"], case["H"], case["k"], case["ratio"]
    kv, od = case.get("kv", O.BF16), case.get("out", O.BF16)
    ns = len(case["pos"])
    max_pos = max(max(p) for p in case["pos"])
    mb = (max_pos + 256) // 256 + 1
    tail = 3
    first_low = [max(0, max(p) // 256 - 1) for p in case["pos"]]
    bt = tail_table(seed, ns, mb, first_low, tail)
    P, P_low = ns * mb, ns * tail
    per_page = 256 // r

    def kv_rows(tid, n):
        if kv == O.FP8:
            return fp8_random_rows(seed, tid, n, D)
        return randn_bf16(seed, tid, (n, D)).view(np.uint8).reshape(n, -1)

    main = O.HostPool(r, case["coff"], D, R, THETA, kv, P, state=True)
    for s_ in range(ns):
        scatter_rows(main.rows, bt, s_, r, kv_rows(40 + 2 * s_, per_page * mb))
    raw = O.HostPool(1, 1, D, R, THETA, kv, P_low, state=False)
    for s_ in range(ns):
        scatter_rows(raw.rows, bt, s_, 1, kv_rows(100 + 2 * s_, 256 * tail), i0=256 * first_low[s_])
    main.state_x[:P_low] = randn_bf16(seed, 13, main.state_x[:P_low].shape)
    main.state_logits[:P_low] = randn_f32(seed, 14, main.state_logits[:P_low].shape).astype(np.float32)
    q_seq = np.concatenate([[s_] * len(p) for s_, p in enumerate(case["pos"])]).astype(np.int32)
    q_pos = np.concatenate(case["pos"]).astype(np.int64)
    nq = len(q_pos)
    q = randn_bf16(seed, 22, (nq, H, D))
    topk = None
    if k:  # valid distinct ids below each query's visible count, ascending
        rng = np.random.default_rng(seed)
        topk = np.stack([np.sort(rng.choice(int(p) // r, k, replace=False)) for p in q_pos]).astype(np.int32)
    # new tokens: one per sequence, at the query's position (the queries read below it)
    cu = np.arange(ns + 1, dtype=np.int32)
    st = np.array([p[0] for p in case["pos"]], np.int64)
    x = randn_bf16(seed, 30, (ns, D))
    lg = randn_f32(seed, 32, (ns, case["coff"])).astype(np.float32)
    gain = rand_u(seed, 34, (D,), 0.5, 1.5).astype(np.float32)
    scale = D ** -0.5
    odt = {O.F32: torch.float32, O.BF16: torch.bfloat16, O.FP8: torch.uint8}[od]
    outs = []
    for fused in (False, True):
        gr, gm = gpu_pool(csl, raw, state=False), gpu_pool(csl, main)
        out = torch.empty((nq, H, D), dtype=odt, device=DEV)
        scales = torch.zeros((nq, H, D // 64), dtype=torch.float32, device=DEV) if od == O.FP8 else None
        jobs = [(gr, dev_bf16(x), None, None), (gm, dev_bf16(x), dev(lg), dev(gain))]
        gbt = dev(bt)
        gtk = dev(topk) if k else None
        ws = csl.workspace(csl.hybrid_attn_workspace(nq, H, D, r, k, 128, max_pos))
        say(f"hybrid_attn_decode_insert {case['name']} fused={fused} nq {nq}")
        if fused:
            csl.hybrid_attn_decode_insert(gm, gr, gbt, dev(q_seq), dev(q_pos), max_pos, dev_bf16(q), gtk, k, 128,
                                          scale, od, out, jobs, dev(st), dev(cu), scales, ws)
        else:
            csl.compress_insert_multi(jobs, gbt, dev(st), dev(cu))
            csl.hybrid_attn_decode(gm, gr, gbt, dev(q_seq), dev(q_pos), max_pos, dev_bf16(q), gtk, k, 128, scale, od,
                                   out, scales, ws)
        torch.cuda.synchronize()
        assert csl.read_device_error() == 0
        res = [host(out.view(torch.uint8)), host(gr.rows), host(gm.rows), host_u16(gm.state_x), host(gm.state_logits)]
        if od == O.FP8:
            res.append(host(scales))
        outs.append(res)
        if ws is not None:  # the counter block is left zero
            assert not ws[:4096].any().item()
    names = ["out", "raw rows", "main rows", "main state_x", "main state_logits", "out scales"]
    for nm, a, b in zip(names, outs[0], outs[1]):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{case['name']}: {nm} differ"
    # the attention against the oracle on the pre-insert pools (the inserts write only rows
    # and entries no query reads)
    o_out, o_oscale, o64, f = O.hybrid_attn(main, raw, bt, q_seq, q_pos, q, topk=topk, k=k,
                                            swa_window=128, softmax_scale=scale, out_dtype=od)
    assert f == 0
    g_out = outs[1][0]
    if od == O.F32:
        assert_close(g_out.view(np.float32).reshape(o64.shape), o64, what=case["name"])
    elif od == O.BF16:
        assert_close(O.bf16_array_to_f64(g_out.view(np.uint16).reshape(o64.shape)), o64, what=case["name"])
    else:
        assert_fp8_close(orc, g_out.reshape(o64.shape), outs[1][-1], o_out, o_oscale, what=case["name"])


# ---------------------------------------------------------------------------
# hybrid attention
# ---------------------------------------------------------------------------

def fp8_random_rows(seed, tid, n, D):
    """Synthetic fp8 rows: random finite e4m3fn codes and random positive scales."""
    codes = (rand_u(seed, tid, (n, D)) * 256).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] &= 0xFE
    scales = (rand_u(seed, tid + 1, (n, D // 64), 0.5, 1.5) / 128.0).astype(np.float32)
    return np.concatenate([codes, scales.view(np.uint8)], axis=1)


def make_pools(seed, ns, T, D, R, comp_ratio, dtype, with_comp=True):
    mb = T // 256 + 2
    bt = block_table(seed, ns, mb, extra_pages=1)
    np_ = ns * mb + 1
    comp = O.HostPool(comp_ratio, 1, D, R, THETA, dtype, np_, state=False) if with_comp else None
    swa = O.HostPool(1, 1, D, R, THETA, dtype, np_, state=False)
    for s in range(ns):
        n_raw = 256 * mb
        if dtype == O.BF16:
            raw = randn_bf16(seed, 40 + s, (n_raw, D)).view(np.uint8).reshape(n_raw, -1)
        else:
            raw = fp8_random_rows(seed, 40 + 2 * s, n_raw, D)
        scatter_rows(swa.rows, bt, s, 1, raw)
        if with_comp:
            nc = n_raw // comp_ratio
            if dtype == O.BF16:
                cr = randn_bf16(seed, 60 + s, (nc, D)).view(np.uint8).reshape(nc, -1)
            else:
                cr = fp8_random_rows(seed, 60 + 2 * s, nc, D)
            scatter_rows(comp.rows, bt, s, comp_ratio, cr)
    return comp, swa, bt


def random_topk(seed, q_pos, ratio, k, invalid=False):
    rs = np.random.default_rng(seed)
    out = np.full((len(q_pos), k), -1, np.int32)
    for n, p in enumerate(q_pos):
        nv = int(p) // ratio
        m = min(k, nv) if n % 3 else min(k, nv) // 2
        pick = np.sort(rs.choice(nv, size=m, replace=False)) if m else np.zeros(0, np.int32)
        out[n, :m] = pick
    if invalid:
        out[0, -1] = int(q_pos[0]) // ratio + 5   # not visible: masked, flagged
    return out


ATTN_CASES = [
    dict(name="c4a_d128_h8_k64_f32", D=128, R=32, H=8, ratio=4, k=64, dtype=O.BF16, out=O.F32,
         pos=[[1, 5, 127, 128, 130, 600, 1023, 1024]]),
    # the 128-dim kernel and the 128-dim combine with bf16 and fp8 output
    dict(name="c4a_d128_h8_k64_bf16", D=128, R=32, H=8, ratio=4, k=64, dtype=O.BF16, out=O.BF16,
         pos=[[1, 5, 127, 128, 130, 600, 1023, 1024]]),
    dict(name="c4a_d128_h8_k64_fp8out", D=128, R=32, H=8, ratio=4, k=64, dtype=O.BF16, out=O.FP8,
         pos=[[2, 64, 129, 700, 1024], [900, 3]]),
    dict(name="c4a_d512_h64_k512_bf16_split", D=512, R=64, H=64, ratio=4, k=512, dtype=O.BF16, out=O.BF16,
         pos=[[2048, 2049, 4099], [3000, 700]]),
    dict(name="c128a_d512_h64_dense_bf16", D=512, R=64, H=64, ratio=128, k=0, dtype=O.BF16, out=O.BF16,
         pos=[[0, 100, 128, 129, 5000, 9000]]),
    dict(name="c4a_d512_h64_fp8kv_fp8out", D=512, R=64, H=64, ratio=4, k=512, dtype=O.FP8, out=O.FP8,
         pos=[[3000, 2500], [4096]]),
    dict(name="c128a_d512_h64_fp8kv_fp8out", D=512, R=64, H=64, ratio=128, k=0, dtype=O.FP8, out=O.FP8,
         pos=[[9000, 130]]),
    dict(name="swa_only_d512_h20_f32", D=512, R=64, H=20, ratio=4, k=0, dtype=O.BF16, out=O.F32,
         pos=[[3, 129, 1000]], no_comp=True),
    dict(name="c4a_d512_h48_invalid_id_bf16", D=512, R=64, H=48, ratio=4, k=64, dtype=O.BF16, out=O.BF16,
         pos=[[900, 1200]], invalid=True),
    # more keys than one pass of resolved addresses holds (1171 entries + 128 raw in one prefill split)
    dict(name="c128a_d512_h64_dense_bf16_long", D=512, R=64, H=64, ratio=128, k=0, dtype=O.BF16, out=O.FP8,
         pos=[[150000, 140001]]),
    # fp8 keys in the 512-dim kernel: bf16 and f32 outputs, heads not a multiple of 32,
    # two key passes, window keys only
    dict(name="c4a_d512_h40_fp8kv_bf16out", D=512, R=64, H=40, ratio=4, k=512, dtype=O.FP8, out=O.BF16,
         pos=[[3000, 2049], [4100]]),
    dict(name="c128a_d512_h64_fp8kv_f32_long", D=512, R=64, H=64, ratio=128, k=0, dtype=O.FP8, out=O.F32,
         pos=[[150000, 131000]]),
    dict(name="swa_only_d512_h64_fp8kv_fp8out", D=512, R=64, H=64, ratio=4, k=0, dtype=O.FP8, out=O.FP8,
         pos=[[5, 129, 1000]], no_comp=True),
    # decode splits: at least as many splits as heads, and 32 queries x 10 splits
    # (more workgroups than compute units)
    dict(name="c128a_d512_h16_splits_over_heads_bf16", D=512, R=64, H=16, ratio=128, k=0, dtype=O.BF16, out=O.BF16,
         pos=[[150000]]),
    dict(name="c4a_d512_h64_k512_32q_fp8out", D=512, R=64, H=64, ratio=4, k=512, dtype=O.BF16, out=O.FP8,
         pos=[[2100 + 37 * i for i in range(16)], [2500 + 53 * i for i in range(16)]]),
    # bf16 keys, more keys than 8 splits of 256 hold: the splits leave partials for the
    # separate combine launch instead of merging in the launch
    dict(name="c128a_d512_h64_dense_bf16_partials_path", D=512, R=64, H=64, ratio=128, k=0, dtype=O.BF16,
         out=O.BF16, pos=[[300000]]),
    # fp8 keys, one query over 2343 + 128 keys: more splits than the launch merges, so
    # the partials go to the combine kernel
    dict(name="c128a_d512_h64_fp8kv_partials_path_bf16out", D=512, R=64, H=64, ratio=128, k=0, dtype=O.FP8,
         out=O.BF16, pos=[[300000]]),
    # 128-dim keys with bf16 and fp8 output (the generic kernel's precision variant and the
    # combine kernel's 128-dim stores)
    dict(name="c4a_d128_h8_k64_bf16out", D=128, R=32, H=8, ratio=4, k=64, dtype=O.BF16, out=O.BF16,
         pos=[[130, 600, 1023, 1024], [700]]),
    dict(name="c4a_d128_h16_k64_fp8out", D=128, R=32, H=16, ratio=4, k=64, dtype=O.BF16, out=O.FP8,
         pos=[[1, 300, 1023], [900, 1024]]),
]


@pytest.mark.parametrize("mode", ["decode", "prefill"])
@pytest.mark.parametrize("case", ATTN_CASES, ids=[c["name"] for c in ATTN_CASES])
def test_hybrid_attn_parity(csl, orc, case, mode):
    D, R, H, ratio, k, dt, od = case["D"], case["R"], case["H"], case["ratio"], case["k"], case["dtype"], case["out"]
    seed = zlib.crc32(case["name"].encode()) % 1000
    pos_lists = case["pos"]
    if mode == "prefill":  # prefill queries of a sequence are consecutive positions
        pos_lists = [list(range(p[0], p[0] + len(p))) for p in pos_lists]
    ns = len(pos_lists)
    max_pos = max(max(p) for p in pos_lists)
    comp, swa, bt = make_pools(seed, ns, max_pos, D, R, ratio, dt, with_comp=not case.get("no_comp"))
    q_seq = np.concatenate([[s] * len(p) for s, p in enumerate(pos_lists)]).astype(np.int32)
    q_pos = np.concatenate(pos_lists).astype(np.int64)
    nq = len(q_pos)
    q = randn_bf16(seed, 80, (nq, H, D))
    topk = random_topk(seed, q_pos, ratio, k, case.get("invalid", False)) if k else None
    scale = D ** -0.5
    o_out, o_sc, o64, f = O.hybrid_attn(comp, swa, bt, q_seq, q_pos, q, topk=topk, k=k, swa_window=128,
                                        softmax_scale=scale, out_dtype=od)
    assert f == (1 if case.get("invalid") else 0)
    gcomp = gpu_pool(csl, comp, state=False) if comp is not None else None
    gswa = gpu_pool(csl, swa, state=False)
    odt = {O.F32: torch.float32, O.BF16: torch.bfloat16, O.FP8: torch.uint8}[od]
    out = torch.empty((nq, H, D), dtype=odt, device=DEV)
    scales = torch.empty((nq, H, D // 64), dtype=torch.float32, device=DEV) if od == O.FP8 else None
    gtopk = dev(topk) if topk is not None else None
    say(f"hybrid_attn {mode} {case['name']} nq {nq}")
    if mode == "decode":
        wsb = csl.hybrid_attn_workspace(nq, H, D, ratio if comp is not None else 0, k, 128, max_pos)
        ws = torch.zeros(max(1, wsb // 4), dtype=torch.float32, device=DEV)
        csl.hybrid_attn_decode(gcomp, gswa, dev(bt), dev(q_seq), dev(q_pos), max_pos, dev_bf16(q), gtopk, k, 128,
                               scale, od, out, scales, ws)
    else:
        cu = np.concatenate([[0], np.cumsum([len(p) for p in pos_lists])]).astype(np.int32)
        starts = np.array([p[0] for p in pos_lists], np.int64)
        csl.hybrid_attn_prefill(gcomp, gswa, dev(bt), dev(cu), dev(starts), max_pos, dev_bf16(q), gtopk, k, 128,
                                scale, od, out, scales)
    torch.cuda.synchronize()
    flags = csl.read_device_error()
    assert flags == (csl.DEVERR_TOPK_ID if case.get("invalid") else 0)
    if od == O.F32:
        assert_close(host(out), o64, what=case["name"])
    elif od == O.BF16:
        assert_close(O.bf16_array_to_f64(host_u16(out)), o64, what=case["name"])
    else:
        assert_fp8_close(orc, host(out), host(scales), o_out, o_sc, what=case["name"])


def test_unmapped_page_is_masked_and_flagged(csl, orc):
    D, R, H = 512, 64, 16
    comp, swa, bt = make_pools(7, 1, 1000, D, R, 4, O.BF16)
    bt = bt.copy()
    bt[0, 3] = -1          # positions 768..1023: raw tokens 872..999 partly, entries 192..255
    q_pos = np.array([1000], np.int64)
    q = randn_bf16(7, 80, (1, H, D))
    topk = np.array([[1, 50, 200, 240, -1]], np.int32)
    _, _, o64, f = O.hybrid_attn(comp, swa, bt, [0], q_pos, q, topk=topk, out_dtype=O.F32)
    assert f > 0
    out = torch.empty((1, H, D), dtype=torch.float32, device=DEV)
    ws = torch.zeros(max(1, csl.hybrid_attn_workspace(1, H, D, 4, 5, 128, 1000) // 4), dtype=torch.float32,
                     device=DEV)
    say("unmapped page masked")
    csl.hybrid_attn_decode(gpu_pool(csl, comp, False), gpu_pool(csl, swa, False), dev(bt), dev(np.zeros(1, np.int32)),
                           dev(q_pos), 1000, dev_bf16(q), dev(topk), 5, 128, D ** -0.5, O.F32, out, None, ws)
    torch.cuda.synchronize()
    assert csl.read_device_error() == csl.DEVERR_UNMAPPED_PAGE
    assert_close(host(out), o64, what="unmapped")


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_nan_key_gives_nan_codes_only_where_seen(csl, orc, mode):
    """A NaN in one raw key row makes every output of a query whose window holds that
    row NaN (the fp8 NaN code, either sign), as in the oracle; the other queries stay
    finite and match.  This covers the fp8 epilogue's non-finite path."""
    D, R, H, k = 512, 64, 64, 64
    comp, swa, bt = make_pools(31, 2, 1300, D, R, 4, O.BF16)
    row = gather_rows(swa.rows, bt, 0, 1, 995, 1)
    row.view(np.uint16)[0, 7] = 0x7FC0     # bf16 NaN in dim 7 of raw token 995 of sequence 0
    scatter_rows(swa.rows, bt, 0, 1, row, i0=995)
    pos_lists = [[1000, 1200], [1000]] if mode == "decode" else [[1000, 1001, 1002], [1000, 1001]]
    q_seq = np.concatenate([[s] * len(p) for s, p in enumerate(pos_lists)]).astype(np.int32)
    q_pos = np.concatenate(pos_lists).astype(np.int64)
    nq = len(q_pos)
    q = randn_bf16(31, 80, (nq, H, D))
    topk = random_topk(31, q_pos, 4, k)
    o_out, o_sc, o64, f = O.hybrid_attn(comp, swa, bt, q_seq, q_pos, q, topk=topk, k=k, swa_window=128,
                                        softmax_scale=D ** -0.5, out_dtype=O.FP8)
    assert f == 0
    seen = np.isnan(o64)
    sees = (q_seq == 0) & (q_pos - 995 < 128)
    assert np.array_equal(seen.all(axis=(1, 2)), sees) and not seen[~sees].any()
    out = torch.empty((nq, H, D), dtype=torch.uint8, device=DEV)
    scales = torch.empty((nq, H, D // 64), dtype=torch.float32, device=DEV)
    say(f"nan key {mode} nq {nq}")
    if mode == "decode":
        ws = torch.zeros(max(1, csl.hybrid_attn_workspace(nq, H, D, 4, k, 128, 1200) // 4), dtype=torch.float32,
                         device=DEV)
        csl.hybrid_attn_decode(gpu_pool(csl, comp, False), gpu_pool(csl, swa, False), dev(bt), dev(q_seq),
                               dev(q_pos), 1200, dev_bf16(q), dev(topk), k, 128, D ** -0.5, O.FP8, out, scales, ws)
    else:
        cu = np.array([0, 3, 5], np.int32)
        csl.hybrid_attn_prefill(gpu_pool(csl, comp, False), gpu_pool(csl, swa, False), dev(bt), dev(cu),
                                dev(np.array([1000, 1000], np.int64)), 1002, dev_bf16(q), dev(topk), k, 128,
                                D ** -0.5, O.FP8, out, scales)
    torch.cuda.synchronize()
    assert csl.read_device_error() == 0
    codes = host(out)
    assert np.array_equal((codes & 0x7F) == 0x7F, seen)
    assert np.all(host(scales)[sees] == 1.0) and np.all(o_sc[sees] == 1.0)
    assert_fp8_close(orc, codes[~sees], host(scales)[~sees], o_out[~sees], o_sc[~sees], what="nan key, unseen")


# ---------------------------------------------------------------------------
# the tiny workload end to end (compress x3 -> index_topk -> decode)
# ---------------------------------------------------------------------------

def test_tiny_workload_end_to_end(csl, orc):
    from synth import workloads as W
    w = W.tiny()
    T, D, R, H, HI, DI, k = w.total_tokens, w.dim, w.rope_dims, w.n_heads, w.idx_heads, w.idx_dim, w.topk
    bt = W.block_table(w).numpy()
    from tests.util import bf16_np
    x = bf16_np(W.latent(w, 0, 0, T))
    lg = W.logits(w, 0, 0, T, 2).numpy()
    xi = bf16_np(W.latent(w, 0, 0, T, dim=DI, tid=W.T_XI))
    lgi = W.logits(w, 0, 0, T, 2, tid=W.T_LOGITS_I).numpy()
    qd = W.queries(w)
    q, qi, wi = bf16_np(qd["q"]), bf16_np(qd["q_idx"]), qd["w_idx"].numpy()
    q_pos = w.query_positions().numpy()
    q_seq = w.query_seqs().numpy()
    nq = len(q_pos)
    P = w.num_pages
    o_main = O.HostPool(4, 2, D, R, THETA, O.BF16, P)
    o_idx = O.HostPool(4, 2, DI, 0, THETA, O.BF16, P)
    o_raw = O.HostPool(1, 1, D, R, THETA, O.BF16, P)
    for pool, xx, ll in ((o_main, x, lg), (o_idx, xi, lgi), (o_raw, x, None)):
        assert O.compress_insert(pool, bt, [0], [0, T], xx, ll) == 0
    o_topk, o_kth, o_sc, _ = O.index_topk(o_idx, bt, q_seq, q_pos, qi, wi, k, want_scores=True, max_cand=T // 4)
    g_main = csl.Pool(4, 2, D, R, THETA, csl.BF16, P)
    g_idx = csl.Pool(4, 2, DI, 0, THETA, csl.BF16, P)
    g_raw = csl.Pool(1, 1, D, R, THETA, csl.BF16, P)
    gbt, st, cu = dev(bt), dev(np.zeros(1, np.int64)), dev(np.array([0, T], np.int32))
    say("tiny workload: compress x3")
    csl.compress_insert(g_main, gbt, st, cu, dev_bf16(x), dev(lg))
    csl.compress_insert(g_idx, gbt, st, cu, dev_bf16(xi), dev(lgi))
    csl.compress_insert(g_raw, gbt, st, cu, dev_bf16(x))
    topk = torch.empty((nq, k), dtype=torch.int32, device=DEV)
    ws = torch.empty(csl.index_topk_workspace(nq, T, k) // 4, dtype=torch.float32, device=DEV)
    say("tiny workload: index_topk")
    csl.index_topk(g_idx, gbt, dev(q_seq), dev(q_pos), T, dev_bf16(qi), dev(wi), k, topk, None, ws)
    out = torch.empty((nq, H, D), dtype=torch.float32, device=DEV)
    wsa = torch.zeros(max(1, csl.hybrid_attn_workspace(nq, H, D, 4, k, w.swa, T) // 4), dtype=torch.float32,
                      device=DEV)
    say("tiny workload: hybrid_attn_decode")
    csl.hybrid_attn_decode(g_main, g_raw, gbt, dev(q_seq), dev(q_pos), T, dev_bf16(q), topk, k, w.swa, D ** -0.5,
                           O.F32, out, None, wsa)
    torch.cuda.synchronize()
    assert csl.read_device_error() == 0
    g_topk = host(topk)
    assert_topk_equivalent(g_topk, o_topk, o_sc, o_kth, what="tiny")
    # every query's attention against the oracle's over the GPU's ids (the oracle's up to allowed swaps)
    _, _, o64g, f = O.hybrid_attn(o_main, o_raw, bt, q_seq, q_pos, q, topk=g_topk, swa_window=w.swa, out_dtype=O.F32)
    assert f == 0
    assert_close(host(out), o64g, what="tiny attention")

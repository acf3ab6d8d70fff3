"""csl_index_attn_decode_noalloc against csl_index_attn_decode.

The no-allocation variant runs the same kernels on the library's static
scratch, so its results must equal those of the workspace call bit for bit.
Two no-allocation calls run back to back, the second on a smaller input (the
scratch keeps the first call's contents); then the workspace calls on fresh
copies of the same pools, and every output and pool is compared.  A call
whose scratch need exceeds the static scratch is refused on the host.
"""
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def make_case(csl, seed, pos, H, HI, DI, out_dtype, with_jobs):
    """Seeded random pools, block table, queries and new tokens (one per sequence, at the
    position of its first query) for decode queries at positions `pos` (one list per sequence)."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    D, R = 512, 64
    ns = len(pos)
    max_pos = max(max(p) for p in pos)
    mb = (max_pos + 256) // 256 + 1
    P = ns * mb
    bt = torch.randperm(P, generator=g, device=DEV).to(torch.int32).reshape(ns, mb).contiguous()

    def rnd_bf16(*shape):
        return torch.randn(*shape, generator=g, device=DEV).to(torch.bfloat16)

    idx = dict(ratio=4, coff=2, dim=DI, rope=0, rows=rnd_bf16(P, 64, DI).view(torch.uint8))
    main = dict(ratio=4, coff=2, dim=D, rope=R, rows=rnd_bf16(P, 64, D).view(torch.uint8))
    raw = dict(ratio=1, coff=1, dim=D, rope=R, rows=rnd_bf16(P, 256, D).view(torch.uint8))
    for p in (idx, main):
        p["state_x"] = rnd_bf16(P, 256, p["dim"]) if with_jobs else None
        p["state_logits"] = torch.randn(P, 256, 2, generator=g, device=DEV) if with_jobs else None
    q_seq = torch.tensor([s for s, p in enumerate(pos) for _ in p], dtype=torch.int32, device=DEV)
    q_pos = torch.tensor([x for p in pos for x in p], dtype=torch.int64, device=DEV)
    nq = int(q_pos.numel())
    case = dict(pools=(idx, main, raw), bt=bt, q_seq=q_seq, q_pos=q_pos, max_pos=max_pos, nq=nq, H=H,
                out_dtype=out_dtype, with_jobs=with_jobs,
                qi=rnd_bf16(nq, HI, DI), w=torch.rand(nq, HI, generator=g, device=DEV), q=rnd_bf16(nq, H, D),
                st=torch.tensor([p[0] for p in pos], dtype=torch.int64, device=DEV),
                cu=torch.tensor([0] + list(range(1, ns + 1)), dtype=torch.int32, device=DEV),
                x=rnd_bf16(ns, D), xi=rnd_bf16(ns, DI), lg=torch.randn(ns, 2, generator=g, device=DEV),
                li=torch.randn(ns, 2, generator=g, device=DEV),
                gain=0.5 + torch.rand(D, generator=g, device=DEV))
    return case


def run(csl, case, noalloc, max_pos=None):
    """One fused decode call on fresh copies of the case's pools; returns the tensors it writes."""
    k, swa = 512, 128
    pools = []
    for p in case["pools"]:
        pools.append(csl.Pool(p["ratio"], p["coff"], p["dim"], p["rope"], 10000.0, csl.BF16, p["rows"].shape[0],
                              rows=p["rows"].clone(), state=False,
                              state_x=None if p.get("state_x") is None else p["state_x"].clone(),
                              state_logits=None if p.get("state_logits") is None else p["state_logits"].clone()))
    gi, gm, gr = pools
    nq, H, od = case["nq"], case["H"], case["out_dtype"]
    odt = {csl.F32: torch.float32, csl.BF16: torch.bfloat16, csl.FP8: torch.uint8}[od]
    topk = torch.full((nq, k), -7, dtype=torch.int32, device=DEV)
    kth = torch.full((nq,), -7.0, dtype=torch.float32, device=DEV)
    out = torch.full((nq, H, 512), 7, dtype=odt, device=DEV)
    scales = torch.full((nq, H, 8), -7.0, dtype=torch.float32, device=DEV) if od == csl.FP8 else None
    jobs = []
    if case["with_jobs"]:
        jobs = [(gr, case["x"], None, None), (gm, case["x"], case["lg"], case["gain"]),
                (gi, case["xi"], case["li"], None)]
    mp = case["max_pos"] if max_pos is None else max_pos
    ws = None
    if not noalloc:
        ws = csl.workspace(csl.index_attn_decode_workspace(nq, H, mp, k, swa))
    csl.index_attn_decode(gi, gm, gr, case["bt"], case["q_seq"], case["q_pos"], mp, case["qi"], case["w"], k, topk,
                          case["q"], swa, 512 ** -0.5, od, out, scales, jobs, case["st"], case["cu"], kth, ws,
                          noalloc=noalloc)
    res = dict(topk=topk, kth=kth, out=out.view(torch.uint8), raw_rows=gr.rows, main_rows=gm.rows,
               index_rows=gi.rows)
    if case["with_jobs"]:
        res.update(main_sx=gm.state_x, main_sl=gm.state_logits, index_sx=gi.state_x, index_sl=gi.state_logits)
    if scales is not None:
        res["scales"] = scales
    return res


def test_noalloc_equals_workspace_call():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import compressed_sparse_long_amd as csl
    csl.read_device_error()
    # 16 sequences, one query and one new token each (inserts into all three pools), 64 heads;
    # then a smaller call: three queries on two sequences, 48 heads, fp8 output, no inserts
    big = make_case(csl, 11, [[40000 + 1500 * i] for i in range(16)], 64, 16, 128, csl.BF16, True)
    small = make_case(csl, 12, [[9003, 9004], [20000]], 48, 16, 128, csl.FP8, False)
    say("noalloc call 1: 16 queries, 64 heads, inserts")
    na_big = run(csl, big, noalloc=True)
    say("noalloc call 2: 3 queries, 48 heads, fp8 out")
    na_small = run(csl, small, noalloc=True)
    torch.cuda.synchronize()
    assert csl.read_device_error() == 0
    say("workspace calls")
    ws_big = run(csl, big, noalloc=False)
    ws_small = run(csl, small, noalloc=False)
    torch.cuda.synchronize()
    assert csl.read_device_error() == 0
    for name, a, b in (("16 queries", na_big, ws_big), ("3 queries", na_small, ws_small)):
        assert a.keys() == b.keys()
        for key in a:
            assert torch.equal(a[key].view(torch.uint8), b[key].view(torch.uint8)), f"{name}: {key} differ"
        assert (a["topk"] >= 0).all().item(), f"{name}: top-k not written"
    # a third call, back on the large input, still matches (the counters were left zero)
    say("noalloc call 3: 16 queries again")
    na_again = run(csl, big, noalloc=True)
    torch.cuda.synchronize()
    for key in na_again:
        assert torch.equal(na_again[key].view(torch.uint8), ws_big[key].view(torch.uint8)), f"repeat: {key} differ"


def test_noalloc_refuses_oversized_call():
    import compressed_sparse_long_amd as csl
    # 200 queries up to 4M positions need far more than the 64 MiB static scratch
    nq = 200
    assert csl.index_attn_decode_workspace(nq, 64, 1 << 22, 512, 128) > 64 << 20
    case = make_case(csl, 13, [[9003], [9100]], 64, 16, 128, csl.BF16, False)
    case.update(nq=nq, q=torch.zeros(nq, 64, 512, dtype=torch.bfloat16, device=DEV),
                qi=torch.zeros(nq, 16, 128, dtype=torch.bfloat16, device=DEV),
                w=torch.zeros(nq, 16, device=DEV), q_seq=torch.zeros(nq, dtype=torch.int32, device=DEV),
                q_pos=torch.zeros(nq, dtype=torch.int64, device=DEV))
    with pytest.raises(csl.CslError) as e:
        run(csl, case, noalloc=True, max_pos=1 << 22)
    assert e.value.status == -2  # CSL_ERANGE, refused before any launch
    torch.cuda.synchronize()
    assert csl.read_device_error() == 0

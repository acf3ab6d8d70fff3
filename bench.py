#!/usr/bin/env python3
"""Decode-step benchmark of the hybrid compressed-attention path on one MI355X.

A step is one pass of the whole path over one batch: for every sequence the
new token is inserted into the raw-window, c4a-main and c4a-index pools
(compress_insert x3), the indexer picks the causal top-512 (index_topk) and
64-head attention runs over top-512 U the 128-token window with the inverse
RoPE epilogue (hybrid_attn_decode).  Default workload: 16 sequences of 131072
cached tokens (32768 c4a entries each), queries at p = 131072.

Inputs are resident in HBM before timing; every step reads a different one of
R cache replicas (R * 538 MB main + 134 MB index) so that the 256 MB
Infinity Cache cannot serve one step's reads to the next.  Steps are replayed
from HIP graphs (the launch-amortisation the pages describe for decode).

Prints one JSON line (rank 0, N = 1).  The CPU oracle is timed beside it on a
bounded sample of the same workload (cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode queries/s + HBM GB/s, c4a top-k512+SWA128 at 128K ctx, 1 MI355X"
HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
CSRC = os.path.join(ROOT, "compressed_sparse_long_amd", "csrc")
# committed HBM counter runs: (summary json, kernel source file it was taken on)
TRAFFIC = {
    "index_score": (os.path.join(ROOT, "profiles", "index_score_c4a_decode_b16_128k.pmc.json"), "index_topk.hip"),
    "decode_attention": (os.path.join(ROOT, "profiles", "decode_attn_c4a_decode_b16_128k.pmc.json"),
                         "decode_attn.hip"),
    "prefill_attention": (os.path.join(ROOT, "profiles", "attention_prefill_c4a_8k_on_64k.pmc.json"), "attn.hip"),
}
# headers the kernel files include: a change to any of them changes the kernels
KERNEL_HEADERS = ["csl_device.hpp", "csl_kernels.hpp", "csl_select.hpp", "csl_insert.hpp"]


def source_digest(source: str) -> str:
    """sha256 over a kernel source file and the shared kernel headers, in that order."""
    h = hashlib.sha256()
    for f in [source] + KERNEL_HEADERS:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# workload setup (GPU)
# ---------------------------------------------------------------------------

class DecodeSetup:
    """Pools, block table and step inputs of a decode workload, resident on the GPU."""

    def __init__(self, w, replicas: int, device="cuda", side_stream: bool = False, qside: bool = False,
                 fused_inserts: bool = False, fused_call: bool = True):
        import torch

        import compressed_sparse_long_amd as csl
        from synth import workloads as W

        self.w, self.csl, self.torch = w, csl, torch
        self.dev = device
        T, D, R, DI = w.ctx, w.dim, w.rope_dims, w.idx_dim
        P = w.num_pages
        self.bt = W.block_table(w).to(device)
        ns = w.num_seqs
        kv = w.kv_dtype
        self.layers = w.layers
        base = {}
        if "c4a" in w.layers:
            base["main4"] = csl.Pool(4, 2, D, R, w.theta, kv, P, device=device)
            base["idx"] = csl.Pool(4, 2, DI, 0, w.theta, w.idx_dtype, P, device=device)
        if "c128a" in w.layers:
            base["main128"] = csl.Pool(128, 1, D, R, w.theta, kv, P, device=device)
        base["raw"] = csl.Pool(1, 1, D, R, w.theta, kv, P, device=device, state=False)
        zeros = torch.zeros(ns, dtype=torch.int64, device=device)
        t0 = time.time()
        for s in range(ns):
            cu = torch.tensor([0] * (s + 1) + [T] * (ns - s), dtype=torch.int32, device=device)
            x = W.latent(w, s, 0, T, device=device)
            csl.compress_insert(base["raw"], self.bt, zeros, cu, x)
            if "c4a" in w.layers:
                csl.compress_insert(base["main4"], self.bt, zeros, cu, x, W.logits(w, s, 0, T, 2, device=device),
                                    W.gain(w, D, device=device))
                if w.synth_index_keys:
                    keys = W.index_keys(w, s, 0, T // 4, device=device)
                    nb = T // 256
                    rows = base["idx"].rows.view(P, 64, DI * 2)
                    rows[self.bt[s, :nb].long()] = keys.view(torch.uint8).view(nb, 64, DI * 2)
                else:
                    xi = W.latent(w, s, 0, T, dim=DI, tid=W.T_XI, device=device)
                    csl.compress_insert(base["idx"], self.bt, zeros, cu, xi,
                                        W.logits(w, s, 0, T, 2, tid=W.T_LOGITS_I, device=device),
                                        W.gain(w, DI, tid=W.T_GAIN_I, device=device))
            if "c128a" in w.layers:
                csl.compress_insert(base["main128"], self.bt, zeros, cu, x,
                                    W.logits(w, s, 0, T, 1, tid=W.T_LOGITS_128, device=device))
            del x
        torch.cuda.synchronize()
        log(f"cache built in {time.time() - t0:.1f}s")
        # replicas: own rows, shared compressor state
        self.reps = [base]
        for _ in range(replicas - 1):
            r = {}
            for k, p in base.items():
                r[k] = csl.Pool(p.ratio, p.coff, p.dim, p.rope_dims, p.theta, p.dtype, p.num_pages,
                                rows=p.rows.clone(), state=False, state_x=p.state_x, state_logits=p.state_logits)
            self.reps.append(r)
        torch.cuda.synchronize()
        # step inputs: the new token at position T of every sequence, queries at p = T
        self.start = torch.full((ns,), T, dtype=torch.int64, device=device)
        self.cu1 = torch.arange(ns + 1, dtype=torch.int32, device=device)
        self.x_new = torch.stack([W.latent(w, s, T, 1, device=device)[0] for s in range(ns)])
        self.lg_new = torch.stack([W.logits(w, s, T, 1, 2, device=device)[0] for s in range(ns)])
        self.lg128_new = torch.stack([W.logits(w, s, T, 1, 1, tid=W.T_LOGITS_128, device=device)[0]
                                      for s in range(ns)])
        self.xi_new = torch.stack([W.latent(w, s, T, 1, dim=DI, tid=W.T_XI, device=device)[0] for s in range(ns)])
        self.lgi_new = torch.stack([W.logits(w, s, T, 1, 2, tid=W.T_LOGITS_I, device=device)[0] for s in range(ns)])
        self.gain = W.gain(w, D, device=device)
        self.gain_i = W.gain(w, DI, tid=W.T_GAIN_I, device=device)
        qd = W.queries(w, device=device)
        self.q, self.q_idx, self.w_idx = qd["q"], qd["q_idx"], qd["w_idx"]
        self.q_seq = w.query_seqs().to(device)
        self.q_pos = w.query_positions().to(device)
        nq = w.num_q
        self.max_pos = T
        self.topk = torch.empty((nq, w.topk), dtype=torch.int32, device=device)
        self.ws_idx = torch.empty(max(1, csl.index_topk_workspace(nq, T, w.topk) // 4), dtype=torch.float32,
                                  device=device)
        ws4 = csl.hybrid_attn_workspace(nq, w.n_heads, D, 4, w.topk, w.swa, T) if "c4a" in w.layers else 0
        ws128 = csl.hybrid_attn_workspace(nq, w.n_heads, D, 128, 0, w.swa, T) if "c128a" in w.layers else 0
        self.ws_attn = torch.zeros(max(1, max(ws4, ws128) // 4), dtype=torch.float32, device=device)
        # the two-launch step (index scores + inserts, then merge + attention): c4a layers with bf16 keys
        self.fused = fused_call and "c4a" in w.layers
        self.ws_fused = (csl.workspace(csl.index_attn_decode_workspace(nq, w.n_heads, T, w.topk, w.swa), device)
                         if self.fused else None)
        odt = {0: torch.float32, 1: torch.bfloat16, 2: torch.uint8}[w.out_dtype]
        self.out = {l: torch.empty((nq, w.n_heads, D), dtype=odt, device=device) for l in w.layers}
        self.out_scales = {l: (torch.empty((nq, w.n_heads, D // 64), dtype=torch.float32, device=device)
                               if w.out_dtype == 2 else None) for l in w.layers}
        self.scale = D ** -0.5
        self.side = torch.cuda.Stream() if side_stream else None
        # with the query side in the step, q is produced from pre-norm heads by the
        # fused Q norm + RoPE + raw-key insert launch (which then owns the raw insert)
        self.qside = qside
        self.fused_inserts = fused_inserts and not side_stream
        if qside:
            self.q_pre = self.q.clone()
            self.gain_q = W.gain(w, D, tid=W.T_GAIN_Q, device=device)

    def insert_jobs(self, p):
        """The new token's insert into every pool of the layer."""
        jobs = [] if self.qside else [(p["raw"], self.x_new, None, None)]
        if "c4a" in self.layers:
            jobs += [(p["main4"], self.x_new, self.lg_new, self.gain), (p["idx"], self.xi_new, self.lgi_new, self.gain_i)]
        if "c128a" in self.layers:
            jobs += [(p["main128"], self.x_new, self.lg128_new, None)]
        return jobs

    def inserts(self, p):
        """The new token into every pool of the layer, one fused launch."""
        self.csl.compress_insert_multi(self.insert_jobs(p), self.bt, self.start, self.cu1)

    def step(self, r: int):
        """One decode step.  By default (c4a layers) the step is the
        two-launch call index_attn_decode: index scores with the raw and main
        inserts riding in the score launch, then the candidates' merge and the
        attention with the index insert riding in it (the query at p reads
        positions < p only); a dense c128a layer's step is one launch,
        hybrid_attn_decode_insert, whose attention workgroups carry the
        inserts.  With --separate-calls the inserts ride in the
        indexer's top-k launch (index_topk_insert) and attention is its own call;
        or they go first in a launch of their own, or, with side streams, beside
        the indexer and attention, forked from and joined back into the current
        stream."""
        p, torch = self.reps[r], self.torch
        if self.fused_inserts and "c4a" in self.layers:
            self.attend(r, with_inserts=True)
            return
        if self.fused_inserts and tuple(self.layers) == ("c128a",) and not self.qside:
            # the dense step in one launch: the inserts ride in the attention launch
            w = self.w
            self.csl.hybrid_attn_decode_insert(p["main128"], p["raw"], self.bt, self.q_seq, self.q_pos, self.max_pos,
                                               self.q, None, 0, w.swa, self.scale, w.out_dtype, self.out["c128a"],
                                               self.insert_jobs(p), self.start, self.cu1, self.out_scales["c128a"],
                                               self.ws_attn)
            return
        if self.qside:
            self.csl.q_norm_rope_insert(p["raw"], self.bt, self.start, self.cu1, self.x_new, self.q_pre, self.gain_q,
                                        q_out=self.q)
        if self.side is not None:
            main = torch.cuda.current_stream()
            self.side.wait_stream(main)
            with torch.cuda.stream(self.side):
                self.inserts(p)
        else:
            self.inserts(p)
        self.attend(r)
        if self.side is not None:
            torch.cuda.current_stream().wait_stream(self.side)

    def attend(self, r: int, with_inserts: bool = False):
        """The query side of a step: index top-k and attention of every layer
        (with_inserts: the step's inserts in the top-k launch)."""
        csl, w, p = self.csl, self.w, self.reps[r]
        if self.fused:
            qs = (p["raw"], self.x_new, self.q_pre, self.gain_q, self.q) if (with_inserts and self.qside) else None
            csl.index_attn_decode(p["idx"], p["main4"], p["raw"], self.bt, self.q_seq, self.q_pos, self.max_pos,
                                  self.q_idx, self.w_idx, w.topk, self.topk, self.q, w.swa, self.scale, w.out_dtype,
                                  self.out["c4a"], self.out_scales["c4a"],
                                  self.insert_jobs(p) if with_inserts else (), self.start, self.cu1, None,
                                  self.ws_fused, qside=qs)
        elif "c4a" in self.layers:
            if with_inserts:
                qs = (p["raw"], self.x_new, self.q_pre, self.gain_q, self.q) if self.qside else None
                csl.index_topk_insert(p["idx"], self.bt, self.q_seq, self.q_pos, self.max_pos, self.q_idx, self.w_idx,
                                      w.topk, self.topk, self.insert_jobs(p), self.start, self.cu1, None, self.ws_idx,
                                      qside=qs)
            else:
                csl.index_topk(p["idx"], self.bt, self.q_seq, self.q_pos, self.max_pos, self.q_idx, self.w_idx, w.topk,
                               self.topk, None, self.ws_idx)
            csl.hybrid_attn_decode(p["main4"], p["raw"], self.bt, self.q_seq, self.q_pos, self.max_pos, self.q,
                                   self.topk, w.topk, w.swa, self.scale, w.out_dtype, self.out["c4a"],
                                   self.out_scales["c4a"], self.ws_attn)
        if "c128a" in self.layers:
            csl.hybrid_attn_decode(p["main128"], p["raw"], self.bt, self.q_seq, self.q_pos, self.max_pos, self.q,
                                   None, 0, w.swa, self.scale, w.out_dtype, self.out["c128a"],
                                   self.out_scales["c128a"], self.ws_attn)

    def algorithmic_bytes_per_step(self) -> dict:
        """Bytes the method must move per step (no intermediate buffers)."""
        w = self.w
        nq, D, H = w.num_q, w.dim, w.n_heads
        rb = self.csl.row_bytes(D, w.kv_dtype)
        ob = {0: 4 * D, 1: 2 * D, 2: D + 4 * (D // 64)}[w.out_dtype]
        per_q = {}
        qio = H * D * 2 + H * ob + (2 * H * D * 2 if self.qside else 0)
        ins = 2 * D * 2 + rb  # raw insert: x read, state x write (c4a/c128a), raw row write
        if "c4a" in w.layers:
            irb = self.csl.row_bytes(w.idx_dim, w.idx_dtype)
            idx = w.ctx // 4 * irb + w.idx_heads * w.idx_dim * 2 + w.idx_heads * 4
            per_q["index_score"] = idx
            per_q["c4a"] = idx + (w.topk + w.swa) * rb + qio + ins + w.idx_dim * 2 + irb
        if "c128a" in w.layers:
            per_q["c128a"] = (w.ctx // 128 + w.swa) * rb + qio + ins
        return {k: v * nq for k, v in per_q.items()}

    def attention_bytes_per_launch(self, layer: str) -> int:
        """Algorithmic bytes of one attention launch: the gathered key rows, q and the output."""
        w = self.w
        rb = self.csl.row_bytes(w.dim, w.kv_dtype)
        ob = {0: 4 * w.dim, 1: 2 * w.dim, 2: w.dim + 4 * (w.dim // 64)}[w.out_dtype]
        keys = (w.topk if layer == "c4a" else w.ctx // 128) + w.swa
        return w.num_q * (keys * rb + w.n_heads * w.dim * 2 + w.n_heads * ob)


class PrefillSetup:
    """A prefill chunk on one sequence: a prefix built by compress_insert
    (untimed), then the step: the chunk's new tokens into the raw, c4a-main
    and c4a-index pools (one fused launch), the indexer's causal top-k for one
    query per new token, and attention over top-k U window for every query."""

    def __init__(self, w, device="cuda"):
        import torch

        import compressed_sparse_long_amd as csl
        from synth import workloads as W

        assert w.prefill and w.num_seqs == 1 and w.layers == ("c4a",)
        self.w, self.csl, self.torch = w, csl, torch
        T0, n, D, R, DI, P = w.ctx, w.new_tokens, w.dim, w.rope_dims, w.idx_dim, w.num_pages
        self.bt = W.block_table(w).to(device)
        kv = w.kv_dtype
        self.raw = csl.Pool(1, 1, D, R, w.theta, kv, P, device=device, state=False)
        self.main = csl.Pool(4, 2, D, R, w.theta, kv, P, device=device)
        self.idx = csl.Pool(4, 2, DI, 0, w.theta, csl.BF16, P, device=device)
        self.gain = W.gain(w, D, device=device)
        self.gain_i = W.gain(w, DI, tid=W.T_GAIN_I, device=device)
        t0 = time.time()
        zero = torch.zeros(1, dtype=torch.int64, device=device)
        cu = torch.tensor([0, T0], dtype=torch.int32, device=device)
        x = W.latent(w, 0, 0, T0, device=device)
        xi = W.latent(w, 0, 0, T0, dim=DI, tid=W.T_XI, device=device)
        csl.compress_insert_multi([(self.raw, x, None, None),
                                   (self.main, x, W.logits(w, 0, 0, T0, 2, device=device), self.gain),
                                   (self.idx, xi, W.logits(w, 0, 0, T0, 2, tid=W.T_LOGITS_I, device=device),
                                    self.gain_i)], self.bt, zero, cu)
        del x, xi
        torch.cuda.synchronize()
        log(f"prefix of {T0} tokens built in {time.time() - t0:.1f}s")
        self.start = torch.full((1,), T0, dtype=torch.int64, device=device)
        self.cu_new = torch.tensor([0, n], dtype=torch.int32, device=device)
        self.x_new = W.latent(w, 0, T0, n, device=device)
        self.lg_new = W.logits(w, 0, T0, n, 2, device=device)
        self.xi_new = W.latent(w, 0, T0, n, dim=DI, tid=W.T_XI, device=device)
        self.lgi_new = W.logits(w, 0, T0, n, 2, tid=W.T_LOGITS_I, device=device)
        qd = W.queries(w, device=device)
        self.q, self.q_idx, self.w_idx = qd["q"], qd["q_idx"], qd["w_idx"]
        self.q_seq = w.query_seqs().to(device)
        self.q_pos = w.query_positions().to(device)
        self.max_pos = T0 + n - 1
        nq = w.num_q
        self.topk = torch.empty((nq, w.topk), dtype=torch.int32, device=device)
        self.ws_idx = torch.empty(max(1, csl.index_topk_workspace(nq, self.max_pos, w.topk) // 4),
                                  dtype=torch.float32, device=device)
        odt = {0: torch.float32, 1: torch.bfloat16, 2: torch.uint8}[w.out_dtype]
        self.out = torch.empty((nq, w.n_heads, D), dtype=odt, device=device)
        self.out_scales = (torch.empty((nq, w.n_heads, D // 64), dtype=torch.float32, device=device)
                           if w.out_dtype == 2 else None)
        self.scale = D ** -0.5

    def step(self):
        csl, w = self.csl, self.w
        csl.compress_insert_multi([(self.raw, self.x_new, None, None),
                                   (self.main, self.x_new, self.lg_new, self.gain),
                                   (self.idx, self.xi_new, self.lgi_new, self.gain_i)], self.bt, self.start,
                                  self.cu_new)
        self.index()
        self.attend()

    def index(self):
        self.csl.index_topk(self.idx, self.bt, self.q_seq, self.q_pos, self.max_pos, self.q_idx, self.w_idx,
                            self.w.topk, self.topk, None, self.ws_idx)

    def attend(self):
        csl, w = self.csl, self.w
        csl.hybrid_attn_prefill(self.main, self.raw, self.bt, self.cu_new, self.start, self.max_pos, self.q,
                                self.topk, w.topk, w.swa, self.scale, w.out_dtype, self.out, self.out_scales)

    def algorithmic_flops(self) -> dict:
        """Multiply-adds x 2 the method must do: indexer over every visible entry
        of every query, attention (QK and PV) over top-k U window keys."""
        w = self.w
        pos = w.query_positions()
        vis = (pos // 4).clamp(min=0)
        keys = vis.clamp(max=w.topk) + pos.clamp(max=w.swa)
        idx = int(vis.sum()) * w.idx_heads * w.idx_dim * 2
        att = int(keys.sum()) * w.n_heads * w.dim * 2 * 2
        return {"index_score": idx, "attention": att}


# ---------------------------------------------------------------------------
# CPU oracle baseline on a bounded sample of the same workload
# ---------------------------------------------------------------------------

def cpu_baseline(setup: DecodeSetup, n_seqs: int, seconds: float) -> dict:
    import numpy as np
    import torch

    import oracle as O
    from synth import workloads as W

    w = setup.w
    assert w.layers == ("c4a",), "the CPU baseline covers the c4a decode workload"
    T, D, R, DI = w.ctx, w.dim, w.rope_dims, w.idx_dim
    n = min(n_seqs, w.num_seqs)
    mb = w.max_blocks
    bt = np.arange(n * mb, dtype=np.int32).reshape(n, mb)
    P = n * mb
    t0 = time.time()
    main = O.HostPool(4, 2, D, R, w.theta, O.BF16, P)
    raw = O.HostPool(1, 1, D, R, w.theta, O.BF16, P)
    idx = O.HostPool(4, 2, DI, 0, w.theta, O.FP4 if w.idx_dtype == 3 else O.BF16, P)

    def u16(t):
        return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)

    xs = np.concatenate([u16(W.latent(w, s, 0, T, device="cuda")) for s in range(n)])
    lgs = np.concatenate([W.logits(w, s, 0, T, 2, device="cuda").cpu().numpy() for s in range(n)])
    st = np.zeros(n, np.int64)
    cu = (np.arange(n + 1) * T).astype(np.int32)
    assert O.compress_insert(main, bt, st, cu, xs, lgs) == 0
    assert O.compress_insert(raw, bt, st, cu, xs) == 0
    del xs, lgs
    if w.synth_index_keys:
        for s in range(n):
            keys = u16(W.index_keys(w, s, 0, T // 4, device="cuda"))
            idx.rows[bt[s, :T // 256]] = keys.view(np.uint8).reshape(T // 256, 64, DI * 2)
    else:
        xis = np.concatenate([u16(W.latent(w, s, 0, T, dim=DI, tid=W.T_XI, device="cuda")) for s in range(n)])
        lis = np.concatenate([W.logits(w, s, 0, T, 2, tid=W.T_LOGITS_I, device="cuda").cpu().numpy()
                              for s in range(n)])
        assert O.compress_insert(idx, bt, st, cu, xis, lis) == 0
        del xis, lis
    log(f"oracle cache for {n} sequences built in {time.time() - t0:.1f}s")
    x_new = u16(setup.x_new[:n])
    lg_new = setup.lg_new[:n].cpu().numpy()
    xi_new = u16(setup.xi_new[:n])
    lgi_new = setup.lgi_new[:n].cpu().numpy()
    q = u16(setup.q[:n])
    qi = u16(setup.q_idx[:n])
    wi = setup.w_idx[:n].cpu().numpy()
    q_seq = np.arange(n, dtype=np.int32)
    q_pos = np.full(n, T, np.int64)
    st1 = np.full(n, T, np.int64)
    cu1 = np.arange(n + 1, dtype=np.int32)
    def run(secs):
        reps, t_start = 0, time.perf_counter()
        while True:
            O.compress_insert(raw, bt, st1, cu1, x_new)
            O.compress_insert(main, bt, st1, cu1, x_new, lg_new)
            O.compress_insert(idx, bt, st1, cu1, xi_new, lgi_new)
            topk, _, _, _ = O.index_topk(idx, bt, q_seq, q_pos, qi, wi, w.topk)
            O.hybrid_attn(main, raw, bt, q_seq, q_pos, q, topk=topk, swa_window=w.swa, softmax_scale=setup.scale,
                          out_dtype=w.out_dtype)
            reps += 1
            el = time.perf_counter() - t_start
            if el >= secs:
                return reps, el

    threads = O.num_threads()
    reps, el = run(seconds)
    O.set_threads(1)
    reps1, el1 = run(seconds / 4)
    O.set_threads(threads)
    model = ""
    try:
        model = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": round(n * reps / el, 3), "unit": "queries/s", "cores": min(threads, n), "kind": "oracle",
            "sample": f"{n} of the {w.num_seqs} sequences (one query each) x {reps} full decode steps "
                      f"(compress_insert x3, index_topk, hybrid_attn) in {el:.1f}s, fp64, OpenMP over queries "
                      f"({threads} threads available)",
            "one_thread_value": round(n * reps1 / el1, 3), "cpu_model": model, "nproc": os.cpu_count(),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def cpu_baseline_prefill(w, n_sample: int, seconds: float, device="cuda") -> dict:
    """The oracle on the prefill chunk: the prefix cache is built untimed; then the
    chunk's inserts (all new tokens, three pools) are timed once, and the index
    top-k plus attention of evenly spaced sampled queries, in batches of 16 (the
    oracle spreads a batch's queries over its threads), for `seconds`.  tokens/s =
    1 / (insert time per token + top-k and attention time per query)."""
    import numpy as np
    import torch

    import oracle as O
    from synth import workloads as W

    T0, n, D, R, DI = w.ctx, w.new_tokens, w.dim, w.rope_dims, w.idx_dim
    mb = w.max_blocks
    bt = np.arange(mb, dtype=np.int32)[None]
    main = O.HostPool(4, 2, D, R, w.theta, w.kv_dtype, mb)
    raw = O.HostPool(1, 1, D, R, w.theta, w.kv_dtype, mb)
    idx = O.HostPool(4, 2, DI, 0, w.theta, O.BF16, mb)

    def u16(t):
        return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)

    gain = W.gain(w, D).numpy()
    gain_i = W.gain(w, DI, tid=W.T_GAIN_I).numpy()

    def inputs(t0, cnt):
        return (u16(W.latent(w, 0, t0, cnt, device=device)), W.logits(w, 0, t0, cnt, 2, device=device).cpu().numpy(),
                u16(W.latent(w, 0, t0, cnt, dim=DI, tid=W.T_XI, device=device)),
                W.logits(w, 0, t0, cnt, 2, tid=W.T_LOGITS_I, device=device).cpu().numpy())

    def insert(t0, cnt, x, lg, xi, lgi):
        st, cu = np.array([t0], np.int64), np.array([0, cnt], np.int32)
        assert O.compress_insert(raw, bt, st, cu, x) == 0
        assert O.compress_insert(main, bt, st, cu, x, lg, gain) == 0
        assert O.compress_insert(idx, bt, st, cu, xi, lgi, gain_i) == 0

    t_build = time.time()
    insert(0, T0, *inputs(0, T0))
    log(f"oracle prefix of {T0} tokens built in {time.time() - t_build:.1f}s")
    new = inputs(T0, n)
    t_ins = time.perf_counter()
    insert(T0, n, *new)
    t_ins = time.perf_counter() - t_ins
    qd = W.queries(w, device=device)
    q, qi, wi = u16(qd["q"]), u16(qd["q_idx"]), qd["w_idx"].cpu().numpy()
    pos = w.query_positions().numpy()
    order = np.linspace(0, n - 1, max(16, n_sample)).astype(np.int64)
    scale = D ** -0.5

    def run(secs):
        done, t_start, b = 0, time.perf_counter(), 0
        while True:
            js = order[(16 * b + np.arange(16)) % len(order)]
            b += 1
            seqs = np.zeros(16, np.int32)
            topk, _, _, _ = O.index_topk(idx, bt, seqs, pos[js], qi[js], wi[js], w.topk)
            O.hybrid_attn(main, raw, bt, seqs, pos[js], q[js], topk=topk, swa_window=w.swa, softmax_scale=scale,
                          out_dtype=w.out_dtype)
            done += 16
            el = time.perf_counter() - t_start
            if el >= secs:
                return done, el

    threads = O.num_threads()
    done, el = run(seconds)
    O.set_threads(1)
    done1, el1 = run(seconds / 4)
    O.set_threads(threads)
    per_tok = t_ins / n
    return {"value": round(1.0 / (per_tok + el / done), 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"insert of all {n} new tokens (3 pools) in {t_ins:.1f}s, then index_topk + hybrid_attn of "
                      f"{done} queries (batches of 16 of {len(order)} evenly spaced ones) in {el:.1f}s; fp64, "
                      f"OpenMP over a batch's queries",
            "one_thread_value": round(1.0 / (per_tok + el1 / done1), 1), "nproc": os.cpu_count()}


# ---------------------------------------------------------------------------

def traffic_from_profile(kernel: str, launch_kind: str):
    """HBM bytes per launch of `kernel` from committed rocprofv3 counter runs, or None
    when there are none for this launch or the kernel source changed since."""
    path, source = TRAFFIC[kernel]
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("source_sha256") != source_digest(source) or d.get("launch") != launch_kind:
        return None
    return float(d["hbm_bytes_per_launch"])


def copy_calibration(mb: int, iters: int):
    """A plain elementwise kernel (negation: one fp32 read and one write per
    element) over `mb` MiB, for scaling the HBM byte counters."""
    import torch
    n = mb * (1 << 20)
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(iters):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"kernel": "neg", "read_bytes": n, "write_bytes": n, "iters": iters}))


def probe():
    """Ceilings of this GPU as plain library kernels reach them: a 4 GiB
    device-to-device copy (read + write bytes / time), a sum over the same
    4 GiB (read bytes / time) and a bf16 GEMM of 8192^3 (2 * 8192^3 flops /
    time), each the median of 20 timed runs."""
    import torch
    res = {}
    n = 1 << 30  # fp32 elements: 4 GiB per buffer
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)

    def med(fn, reps=20):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return sorted(ts)[len(ts) // 2]
    t = med(lambda: dst.copy_(src))
    res["copy_GBps"] = round(2 * 4 * n / t / 1e9, 1)
    t = med(lambda: torch.sum(src))
    res["read_GBps"] = round(4 * n / t / 1e9, 1)
    del src, dst
    torch.cuda.empty_cache()
    m = 8192
    a = torch.randn(m, m, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(m, m, dtype=torch.bfloat16, device="cuda")
    t = med(lambda: torch.matmul(a, b))
    res["bf16_gemm_TFLOPs"] = round(2 * m ** 3 / t / 1e12, 1)
    res["peaks"] = {"hbm_GBps": HBM_PEAK_GBPS, "bf16_mfma_TFLOPs": BF16_MFMA_PEAK_TFLOPS}
    print(json.dumps(res), flush=True)


def run_prefill(args):
    """Prefill chunk: steps launched eagerly (milliseconds each, launch cost is
    noise) with every library kernel timed by its own start/end stamps."""
    import torch

    import compressed_sparse_long_amd as csl
    from synth import workloads as W

    w = W.prefill()
    setup = PrefillSetup(w)
    log(f"workload {w.name}: {w.new_tokens} new tokens on a {w.ctx}-token prefix")
    K, warm = args.steps, args.warmup
    for _ in range(warm):
        setup.step()
    torch.cuda.synchronize()
    assert csl.read_device_error() == 0, "device error flags after warm-up"
    kids = {"compress_insert": csl.KERNEL_COMPRESS, "index_score": csl.KERNEL_INDEX_SCORE,
            "topk_select": csl.KERNEL_TOPK_SELECT, "attention": csl.KERNEL_ATTN}
    for k in kids.values():
        csl.timer_read(k)
        csl.timer_enable(k, True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        setup.step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern = {}
    for name, k in kids.items():
        csl.timer_enable(k, False)
        ms, n = csl.timer_read(k)
        kern[name] = {"avg_ms": round(ms / max(1, n), 4), "launches": n}
    assert csl.read_device_error() == 0, "device error flags after the timed steps"
    ms_step = (t1 - t0) * 1e3 / K
    fl = setup.algorithmic_flops()
    for name in ("index_score", "attention"):
        kern[name]["algorithmic_tflop"] = round(fl[name] / 1e12, 2)
        kern[name]["tflops"] = round(fl[name] / (kern[name]["avg_ms"] * 1e-3) / 1e12, 1)
    dom = max(("index_score", "attention"), key=lambda k: kern[k]["avg_ms"])
    ach = kern[dom]["tflops"]
    res = {
        "metric": "prefill tokens/s (c4a layer: insert + indexer top-512 + attention over top-512 U SWA128)",
        "value": round(w.new_tokens / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": warm, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "algorithmic_tflops": round((fl["index_score"] + fl["attention"]) / (ms_step * 1e-3) / 1e12, 1),
        "config": {"workload": w.name, "prefix": w.ctx, "new_tokens": w.new_tokens, "topk": w.topk, "swa": w.swa,
                   "heads": w.n_heads, "latent_dim": w.dim, "indexer": f"{w.idx_heads}x{w.idx_dim}",
                   "kv_dtype": "bf16", "out_dtype": "fp8", "hip_graphs": False},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": ach, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / BF16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": traffic_from_profile("prefill_attention", w.name) if dom == "attention" else None,
                     "timing": "hipExtLaunchKernel start/stop events stamped by each launch in the timed steps"},
        "kernels": kern,
        "cpu_baseline": None if args.no_cpu else cpu_baseline_prefill(w, 256, args.cpu_seconds),
    }
    print(json.dumps(res), flush=True)


def run_qside(args):
    """Query side of a step (per-head Q RMSNorm + Q RoPE, raw-key RoPE + insert,
    one launch) at the decode or the prefill workload's shape: the new tokens'
    64 query heads of 512 (pre-norm, ~N(0,1)) and their raw latent rows."""
    import torch

    import compressed_sparse_long_amd as csl
    from synth import workloads as W

    w = W.c4a_decode() if args.workload == "qside_decode" else W.prefill()
    dev = "cuda"
    ns, n, T, D, H = w.num_seqs, w.new_tokens, w.ctx, w.dim, w.n_heads
    total = ns * n
    bt = W.block_table(w).to(dev)
    raw = csl.Pool(1, 1, D, w.rope_dims, w.theta, w.kv_dtype, w.num_pages, device=dev, state=False)
    start = torch.full((ns,), T, dtype=torch.int64, device=dev)
    cu = torch.arange(ns + 1, dtype=torch.int32, device=dev) * n
    x = torch.cat([W.latent(w, s, T, n, device=dev) for s in range(ns)])
    q = W.queries(w, device=dev)["q"]
    assert q.shape == (total, H, D)
    g = W.gain(w, D, tid=W.T_GAIN_Q, device=dev)
    q_out = torch.empty_like(q)
    log(f"q-side {w.name}: {total} tokens x {H} heads x {D}")

    def launch():
        csl.q_norm_rope_insert(raw, bt, start, cu, x, q, g, q_out=q_out)

    K, warm = args.steps, args.warmup
    for _ in range(warm):
        launch()
    torch.cuda.synchronize()
    assert csl.read_device_error() == 0
    per = 10
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per):
            launch()
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, K // per)
    t0 = time.perf_counter()
    for _ in range(reps):
        graph.replay()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / (reps * per)
    csl.timer_read(csl.KERNEL_QSIDE)
    csl.timer_enable(csl.KERNEL_QSIDE, True)
    for _ in range(min(K, 500)):
        launch()
    torch.cuda.synchronize()
    csl.timer_enable(csl.KERNEL_QSIDE, False)
    k_ms, k_n = csl.timer_read(csl.KERNEL_QSIDE)
    assert csl.read_device_error() == 0
    k_avg = k_ms / max(1, k_n)
    rb = csl.row_bytes(D, w.kv_dtype)
    per_tok = 2 * H * D * 2 + D * 2 + rb
    k_bytes = total * per_tok
    ach = k_bytes / (k_avg * 1e-3) / 1e9
    res = {
        "metric": "query-side tokens/s (per-head Q RMSNorm + RoPE, raw-key RoPE + insert, one launch)",
        "value": round(total / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": reps * per,
        "warmup": warm, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"qside_{w.name}", "tokens": total, "heads": H, "latent_dim": D,
                   "rope_dims": w.rope_dims, "q_gain": g is not None, "hip_graphs": True, "launches_per_graph": per},
        "roofline": {"bound": "hbm", "kernel": "q_norm_rope_insert_kernel", "achieved": round(ach, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": k_bytes, "avg_launch_ms": round(k_avg, 5),
                     "timed_launches": k_n,
                     "timing": "hipExtLaunchKernel start/stop events stamped by each eager launch"},
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        import numpy as np

        import oracle as O
        m = min(total, 256)
        hq = q[:m].cpu().view(torch.int16).numpy().view(np.uint16)
        hx = x[:m].cpu().view(torch.int16).numpy().view(np.uint16)
        hg = None if g is None else g.cpu().numpy()
        hbt = bt.cpu().numpy()
        hp = O.HostPool(1, 1, D, w.rope_dims, w.theta, w.kv_dtype, w.num_pages, state=False)
        seqs = m // n if n > 1 else m
        st = np.full(max(1, seqs), T, np.int64)
        hcu = (np.arange(max(1, seqs) + 1) * (n if n > 1 else 1)).astype(np.int32)
        hcu[-1] = m
        done, t0 = 0, time.perf_counter()
        while True:
            O.q_norm_rope_insert(hp, hbt[:len(st)], st, hcu, hx, hq, hg)
            done += m
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds / 4:
                break
        res["cpu_baseline"] = {"value": round(done / el, 1), "unit": "tokens/s", "cores": O.num_threads(),
                               "kind": "oracle", "sample": f"the first {m} of the step's tokens, repeated for {el:.1f}s"}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="c4a", choices=["c4a", "c4a_fp4", "c128a", "1m", "prefill", "qside_decode", "qside_prefill"])
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--no-graph", action="store_true", help="launch steps eagerly instead of replaying HIP graphs")
    ap.add_argument("--graph-steps", type=int, default=20,
                    help="decode steps per HIP graph (the largest divisor of --steps not above this)")
    ap.add_argument("--timing-steps", type=int, default=200,
                    help="eager steps after the graph replays that time the dominant kernel")
    ap.add_argument("--side-stream", action="store_true",
                    help="run the inserts on a side stream beside the indexer and attention")
    ap.add_argument("--separate-inserts", action="store_true",
                    help="launch the inserts on their own before the indexer instead of inside its top-k launch")
    ap.add_argument("--separate-calls", action="store_true",
                    help="run the c4a step as index_topk_insert + hybrid_attn_decode instead of the two-launch "
                         "index_attn_decode")
    ap.add_argument("--qside", action="store_true",
                    help="start the step from pre-norm query heads: the Q norm + RoPE + raw-key insert (in the top-k "
                         "launch with the other inserts, or its own launch with --separate-inserts) produces q and "
                         "writes the raw key")
    ap.add_argument("--cpu-seqs", type=int, default=16)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--probe", action="store_true",
                    help="only measure this GPU's ceilings: a large device copy (HBM) and a large bf16 GEMM (MFMA)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="only run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the path is data-parallel per sequence (sequences shard across GPUs "
              "with no exchange), and the benchmark runs on a single MI355X; --gpus must be 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration_mb:
        copy_calibration(args.copy_calibration_mb, 10)
        return
    if args.probe:
        probe()
        return

    import torch

    import compressed_sparse_long_amd as csl
    from synth import workloads as W

    if args.workload == "prefill":
        run_prefill(args)
        return
    if args.workload.startswith("qside"):
        run_qside(args)
        return
    w = {"c4a": W.c4a_decode, "c4a_fp4": W.c4a_decode_fp4, "c128a": W.c128a_decode, "1m": W.long_1m}[args.workload]()
    R = max(1, args.replicas)
    setup = DecodeSetup(w, R, side_stream=args.side_stream, qside=args.qside,
                        fused_inserts=not args.separate_inserts,
                        fused_call=not (args.separate_calls or args.separate_inserts or args.side_stream))
    log(f"workload {w.name}: {w.num_seqs} x {w.ctx} tokens, {R} replicas")

    for i in range(args.warmup):
        setup.step(i % R)
    torch.cuda.synchronize()
    assert csl.read_device_error() == 0, "device error flags after warm-up"

    timing_kernel = csl.KERNEL_INDEX_SCORE if "c4a" in w.layers else csl.KERNEL_ATTN
    # every kernel of the step gets its own timer in the eager timing steps
    step_kernels = {"index_score": csl.KERNEL_INDEX_SCORE, "topk_select": csl.KERNEL_TOPK_SELECT,
                    "attention": csl.KERNEL_ATTN, "attn_combine": csl.KERNEL_ATTN_COMBINE}
    if "c4a" not in w.layers:
        step_kernels = {"attention": csl.KERNEL_ATTN, "attn_combine": csl.KERNEL_ATTN_COMBINE}
    graphs = None
    per_graph = 1
    if not args.no_graph:
        # One graph holds G successive steps, step i on cache replica i % R (the replicas stand
        # for successive layers, whose caches are distinct).  A serving engine replays one graph
        # per decode iteration over every layer of the model; replaying a graph costs about 8 us
        # of its own on this GPU, which G steps share.  G is the largest divisor of the timed
        # step count not above --graph-steps, so that exactly K steps are timed.
        per_graph = max(g for g in range(1, max(1, min(args.graph_steps, args.steps)) + 1) if args.steps % g == 0)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(per_graph):
                setup.step(i % R)
        graphs = [g]
        torch.cuda.synchronize()
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()

    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graphs:
        for i in range(K // per_graph):
            graphs[i % len(graphs)].replay()
    else:
        for kid in step_kernels.values():
            csl.timer_enable(kid, True)
        for i in range(K):
            setup.step(i % R)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_dist = None
    if graphs:
        # per-replay durations (HIP events on the replay stream) for the spread
        # of step times; a separate pass, so the timed loop above carries no events
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(min(200, K // per_graph))]
        for i, (e0, e1) in enumerate(evs):
            e0.record()
            graphs[i % len(graphs)].replay()
            e1.record()
        torch.cuda.synchronize()
        us = sorted(e0.elapsed_time(e1) * 1e3 / per_graph for e0, e1 in evs)
        if us:
            q = lambda f: round(us[min(len(us) - 1, int(f * len(us)))], 2)
            step_dist = {"p10": q(0.1), "p50": q(0.5), "p90": q(0.9), "replays": len(us),
                         "timing": f"HIP events around each replay of a {per_graph}-step graph"}
    if graphs:
        # The kernel's own start/end stamps (hipExtLaunchKernel events) are not
        # kept by graph capture, so the dominant kernel's duration comes from
        # eager steps run right after the replays, on the same caches and stream.
        for kid in step_kernels.values():
            csl.timer_enable(kid, True)
        for i in range(args.timing_steps):
            setup.step(i % R)
        torch.cuda.synchronize()
    kern_times = {}
    for name, kid in step_kernels.items():
        csl.timer_enable(kid, False)
        kern_times[name] = csl.timer_read(kid)
    k_ms, k_n = kern_times["index_score" if "c4a" in w.layers else "attention"]
    assert csl.read_device_error() == 0, "device error flags after the timed steps"
    ms_per_step = (t1 - t0) * 1e3 / K
    qps = w.num_q / (ms_per_step * 1e-3)
    alg = setup.algorithmic_bytes_per_step()
    step_bytes = sum(v for k, v in alg.items() if k != "index_score")
    kernel_name = "index_score_kernel" if "c4a" in w.layers else "hybrid_attn_kernel"
    k_avg_ms = k_ms / max(1, k_n)
    k_bytes = alg["index_score"] if "c4a" in w.layers else alg["c128a"]
    achieved = k_bytes / (k_avg_ms * 1e-3) / 1e9 if k_n else None
    roof = {"bound": "hbm", "kernel": kernel_name, "achieved": round(achieved, 1) if achieved else None,
            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4) if achieved else None,
            "traffic": traffic_from_profile("index_score", w.name) if "c4a" in w.layers else None,
            "algorithmic_bytes_per_launch": k_bytes, "avg_launch_ms": round(k_avg_ms, 5), "timed_launches": k_n,
            "timing": ("hipExtLaunchKernel start/stop events stamped by each launch of the kernel itself, over "
                       f"{k_n} eager steps right after the timed graph replays (graph capture drops the stamps)"
                       if graphs else "hipExtLaunchKernel start/stop events stamped by each launch in the timed steps")}
    # one entry per step kernel: average duration, algorithmic bytes per launch and the
    # fraction of the HBM peak they stand for (intermediate buffers are not counted)
    kb = {"index_score": alg.get("index_score", 0),
          # (the 1M workload's attention timer averages its two layers' launches: no byte figure)
          "attention": (0 if len(w.layers) > 1 else setup.attention_bytes_per_launch(w.layers[0])),
          "topk_select": 0, "attn_combine": 0}
    kernels = {}
    for name, (ms, n) in kern_times.items():
        if n == 0:
            continue
        avg = ms / n
        e = {"avg_us": round(avg * 1e3, 2), "launches": n, "algorithmic_bytes_per_launch": kb[name]}
        if kb[name]:
            e["GBps"] = round(kb[name] / (avg * 1e-3) / 1e9, 1)
            e["frac"] = round(kb[name] / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
        if name == "index_score" and "c4a" in w.layers:
            e["traffic"] = traffic_from_profile("index_score", w.name)
        if name == "attention" and setup.fused:
            e["traffic"] = traffic_from_profile("decode_attention", w.name)
        kernels[name] = e
    res = {
        "metric": METRIC, "value": round(qps, 1), "unit": "queries/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.kv_dtype == 1 else "fp8-kv/bf16-mfma", "data": "synthetic",
        "step_us": step_dist,
        "hbm_GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "hbm_frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "context": w.ctx, "layers": list(w.layers),
                   "topk": w.topk, "swa": w.swa, "heads": w.n_heads, "latent_dim": w.dim, "rope_dims": w.rope_dims,
                   "indexer": f"{w.idx_heads}x{w.idx_dim}", "index_dtype": {1: "bf16", 3: "fp4"}[w.idx_dtype],
                   "kv_dtype": {1: "bf16", 2: "fp8"}[w.kv_dtype],
                   "out_dtype": {0: "f32", 1: "bf16", 2: "fp8"}[w.out_dtype], "replicas": R,
                   "hip_graphs": bool(graphs), "steps_per_graph": per_graph, "insert_stream": "side" if args.side_stream else "main",
                   "inserts": ("raw + main in the score launch, index in the attention launch" if setup.fused else
                               "in the top-k launch" if setup.fused_inserts and "c4a" in w.layers else
                               "own launch" + (" (side stream)" if args.side_stream else "")),
                   "query_side_in_step": bool(args.qside),
                   "step_calls": ("index_attn_decode (2 launches)" if setup.fused else
                                  "index_topk_insert + hybrid_attn_decode"),
                   "algorithmic_bytes_per_step": step_bytes},
        "roofline": roof,
        "kernels": kernels,
        "target": ("the decode attention step (index top-k + hybrid attention) at >= 60% of the HBM "
                   "peak: hbm_frac of the whole step; roofline.frac is the score kernel alone"),
    }
    if not args.no_cpu and w.layers == ("c4a",):
        log("timing the CPU oracle")
        res["cpu_baseline"] = cpu_baseline(setup, args.cpu_seqs, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

"""Shapes of the five synthetic workloads and builders of their seeded inputs.

Each workload takes the shapes and value distributions of the pages'
setting (DeepSeek-V4 c4a / c128a layers, 64 MQA heads over a 512-wide shared
latent with 64 RoPE dims, a 16x128 indexer, top-512, a 128-token window,
256-token blocks, contexts up to 1M).  No public benchmark is involved; these
synthetic inputs stand in for the 1M-context serving workloads the pages
describe.

Conventions (the attention method itself lives elsewhere):
  * a decode step for a sequence holding T tokens (positions 0..T-1) inserts
    the new token at position T and runs the query at position p = T;
  * a prefill chunk of n new tokens at positions P..P+n-1 runs one query per
    new token at the token's own position;
  * the block table is a random permutation of all pages, [num_seqs][max_blocks].

Every tensor is a pure function of (seed, tensor id, element index); element
index = row-major position in the full tensor, so slices can be regenerated.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import rng

# tensor ids (stable; changing one changes every derived input)
T_X, T_LOGITS, T_XI, T_LOGITS_I, T_Q, T_QI, T_W, T_GAIN, T_GAIN_I = 1, 2, 3, 4, 5, 6, 7, 8, 9
T_INDEX_KEYS, T_PERM, T_LOGITS_128, T_Q128, T_GAIN_Q = 10, 11, 12, 13, 14
T_ROWS, T_TOPK = 20, 21


@dataclass
class Workload:
    name: str
    seed: int
    num_seqs: int
    ctx: int                 # tokens already cached per sequence before the step
    new_tokens: int          # tokens the step inserts per sequence (decode: 1)
    dim: int = 512
    rope_dims: int = 64
    theta: float = 10000.0
    n_heads: int = 64
    idx_heads: int = 16
    idx_dim: int = 128
    topk: int = 512
    swa: int = 128
    kv_dtype: int = 1        # 1 = bf16 rows, 2 = fp8 rows (64-element groups + fp32 scales)
    idx_dtype: int = 1       # index rows: 1 = bf16, 3 = fp4 (MXFP4: E2M1 codes + E8M0 per 32)
    out_dtype: int = 1       # 0 = f32, 1 = bf16, 2 = fp8
    layers: tuple = ("c4a",)  # "c4a" and/or "c128a"
    synth_index_keys: bool = True   # index cache drawn directly (bf16) instead of compressed
    prefill: bool = False
    gain_range: tuple | None = None  # RMSNorm gain ~U(lo, hi); None = unit gain
    queries: list = field(default_factory=list)  # explicit query positions (tiny workload)

    @property
    def total_tokens(self) -> int:
        return self.ctx + self.new_tokens

    @property
    def max_blocks(self) -> int:
        return (self.total_tokens + 255) // 256

    @property
    def num_pages(self) -> int:
        return self.num_seqs * self.max_blocks

    def query_positions(self) -> torch.Tensor:
        """Position of every query, [num_q] int64 (sequence-major)."""
        if self.queries:
            return torch.tensor(self.queries * self.num_seqs, dtype=torch.int64)
        if self.prefill:
            per = torch.arange(self.ctx, self.ctx + self.new_tokens, dtype=torch.int64)
        else:
            per = torch.tensor([self.ctx], dtype=torch.int64)
        return per.repeat(self.num_seqs)

    def query_seqs(self) -> torch.Tensor:
        per = len(self.queries) if self.queries else (self.new_tokens if self.prefill else 1)
        return torch.arange(self.num_seqs, dtype=torch.int32).repeat_interleave(per)

    @property
    def num_q(self) -> int:
        return int(self.query_positions().numel())


def tiny() -> Workload:
    """Tiny c4a layer: 1 sequence of 1024 tokens, latent [1024,128] with 32 RoPE
    dims, 8 heads, a 4x32 indexer whose keys are compressed from their own
    latent, top-64, window 128, queries at the last 16 positions, fp32 out."""
    return Workload("tiny_c4a_1x1024", seed=0, num_seqs=1, ctx=1024, new_tokens=0, dim=128, rope_dims=32,
                    n_heads=8, idx_heads=4, idx_dim=32, topk=64, out_dtype=0, synth_index_keys=False,
                    queries=list(range(1008, 1024)))


def c128a_decode() -> Workload:
    return Workload("c128a_decode_b8_32k", seed=1, num_seqs=8, ctx=32768, new_tokens=1, layers=("c128a",),
                    topk=0)


def c4a_decode() -> Workload:
    return Workload("c4a_decode_b16_128k_top512_swa128", seed=2, num_seqs=16, ctx=131072, new_tokens=1)


def c4a_decode_fp4() -> Workload:
    """The c4a decode step with the index cache in fp4 (built by the compressor)."""
    return Workload("c4a_decode_b16_128k_top512_swa128_fp4idx", seed=2, num_seqs=16, ctx=131072, new_tokens=1,
                    idx_dtype=3, synth_index_keys=False)


def long_1m() -> Workload:
    return Workload("hybrid_decode_b1_1m_fp8", seed=3, num_seqs=1, ctx=1 << 20, new_tokens=1,
                    layers=("c4a", "c128a"), kv_dtype=2, out_dtype=2)


def prefill() -> Workload:
    return Workload("c4a_prefill_8k_on_64k", seed=4, num_seqs=1, ctx=65536, new_tokens=8192, out_dtype=2,
                    prefill=True, synth_index_keys=False, gain_range=(0.5, 1.5))


ALL = {1: tiny, 2: c128a_decode, 3: c4a_decode, 4: long_1m, 5: prefill}


# ---------------------------------------------------------------------------
# builders
# ---------------------------------------------------------------------------

def block_table(w: Workload) -> torch.Tensor:
    """Random permutation of the workload's pages, [num_seqs][max_blocks] int32."""
    return rng.permutation(w.seed, T_PERM, w.num_pages).to(torch.int32).view(w.num_seqs, w.max_blocks)


def latent(w: Workload, seq: int, t0: int, n: int, dim: int | None = None, tid: int = T_X,
           device="cpu") -> torch.Tensor:
    """Latent tokens t0..t0+n-1 of one sequence, [n][dim] bf16 ~N(0,1)."""
    dim = w.dim if dim is None else dim
    start = (seq * w.total_tokens + t0) * dim
    return rng.normal_bf16(w.seed, tid, n * dim, device, start=start).view(n, dim)


def logits(w: Workload, seq: int, t0: int, n: int, coff: int, tid: int = T_LOGITS, device="cpu") -> torch.Tensor:
    """Per-token compression logits, [n][coff] fp32 ~N(0,1)."""
    start = (seq * w.total_tokens + t0) * coff
    return rng.normal(w.seed, tid, n * coff, device, start=start).view(n, coff)


def gain(w: Workload, dim: int, tid: int = T_GAIN, device="cpu") -> torch.Tensor | None:
    if w.gain_range is None:
        return None
    lo, hi = w.gain_range
    return rng.uniform(w.seed, tid, dim, device, lo, hi).to(torch.float32)


def queries(w: Workload, device="cpu") -> dict:
    """q [num_q][H][D] bf16, q_idx [num_q][H_I][d_I] bf16, w_idx [num_q][H_I] fp32 ~U(0,1)."""
    nq = w.num_q
    return {
        "q": rng.normal_bf16(w.seed, T_Q, nq * w.n_heads * w.dim, device).view(nq, w.n_heads, w.dim),
        "q_idx": rng.normal_bf16(w.seed, T_QI, nq * w.idx_heads * w.idx_dim, device).view(nq, w.idx_heads,
                                                                                          w.idx_dim),
        "w_idx": rng.uniform(w.seed, T_W, nq * w.idx_heads, device).to(torch.float32).view(nq, w.idx_heads),
    }


def index_keys(w: Workload, seq: int, i0: int, n: int, device="cpu") -> torch.Tensor:
    """Directly drawn index-cache entries i0..i0+n-1 of one sequence, [n][d_I] bf16 ~N(0,1)."""
    per_seq = w.total_tokens // 4 + 1
    start = (seq * per_seq + i0) * w.idx_dim
    return rng.normal_bf16(w.seed, T_INDEX_KEYS, n * w.idx_dim, device, start=start).view(n, w.idx_dim)

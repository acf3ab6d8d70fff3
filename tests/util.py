"""Test-side helpers: seeded host arrays, block tables and numpy views of bf16 data."""
from __future__ import annotations

import numpy as np
import torch

from synth import rng

BLOCK = 256


def bf16_np(t: torch.Tensor) -> np.ndarray:
    """bf16 torch tensor -> uint16 numpy array of the same bit patterns."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def randn_bf16(seed: int, tid: int, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return bf16_np(rng.normal_bf16(seed, tid, n)).reshape(shape)


def randn_f32(seed: int, tid: int, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return rng.normal(seed, tid, n).numpy().reshape(shape)


def rand_u(seed: int, tid: int, shape, lo=0.0, hi=1.0) -> np.ndarray:
    n = int(np.prod(shape))
    return rng.uniform(seed, tid, n, lo=lo, hi=hi).numpy().reshape(shape)


def block_table(seed: int, num_seqs: int, max_blocks: int, extra_pages: int = 0, tid: int = 11) -> np.ndarray:
    """Random permutation of num_seqs*max_blocks (+extra) pages, [num_seqs][max_blocks] int32."""
    n = num_seqs * max_blocks + extra_pages
    perm = rng.permutation(seed, tid, n).numpy().astype(np.int32)
    return perm[: num_seqs * max_blocks].reshape(num_seqs, max_blocks).copy()


def page_row(bt: np.ndarray, s: int, i: int, ratio: int):
    """(page, row) of entry i of a ratio-r pool of sequence s."""
    per = BLOCK // ratio
    return int(bt[s, (i * ratio) // BLOCK]), i % per


def scatter_rows(pool_rows: np.ndarray, bt: np.ndarray, s: int, ratio: int, rows: np.ndarray, i0: int = 0):
    """Write dense entry rows [n][row_bytes] of sequence s into a paged pool array."""
    for j in range(rows.shape[0]):
        pg, r = page_row(bt, s, i0 + j, ratio)
        pool_rows[pg, r] = rows[j]


def gather_rows(pool_rows: np.ndarray, bt: np.ndarray, s: int, ratio: int, i0: int, n: int) -> np.ndarray:
    out = np.empty((n, pool_rows.shape[-1]), pool_rows.dtype)
    for j in range(n):
        pg, r = page_row(bt, s, i0 + j, ratio)
        out[j] = pool_rows[pg, r]
    return out


def fp4_rows(orc, vals: np.ndarray) -> np.ndarray:
    """MXFP4 rows [n][row_bytes] of vals [n][d] (float), quantised block by block by the oracle."""
    n, d = vals.shape
    rows = np.zeros((n, orc.row_bytes(d, orc.FP4)), np.uint8)
    for i in range(n):
        for b in range(d // 32):
            codes, sc = orc.mxfp4_block(vals[i, 32 * b:32 * b + 32])
            rows[i, 16 * b:16 * b + 16] = codes
            rows[i, d // 2 + b] = sc
    return rows

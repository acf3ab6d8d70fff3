"""ctypes binding of the plain-C CPU oracle (oracle/csl_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product package
``compressed_sparse_long_amd``.  Arguments are numpy arrays on the host.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csl_oracle.c")
LIB = os.path.join(HERE, "libcsl_oracle.so")

F32, BF16, FP8, FP4 = 0, 1, 2, 3
BLOCK = 256


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (always recompiles)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


class Pool(C.Structure):
    _fields_ = [
        ("ratio", C.c_int32), ("coff", C.c_int32), ("dim", C.c_int32), ("rope_dims", C.c_int32),
        ("rope_theta", C.c_double),
        ("dtype", C.c_int32), ("num_pages", C.c_int32),
        ("rows", C.c_void_p), ("state_x", C.c_void_p), ("state_logits", C.c_void_p),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = C.CDLL(LIB)
        vp, i32, i64, dbl = C.c_void_p, C.c_int32, C.c_int64, C.c_double
        L.csl_oracle_row_bytes.argtypes = [C.c_int, C.c_int]
        L.csl_oracle_row_bytes.restype = i64
        L.csl_oracle_bf16_to_f64.argtypes = [C.c_uint16]
        L.csl_oracle_bf16_to_f64.restype = dbl
        L.csl_oracle_f64_to_bf16.argtypes = [dbl]
        L.csl_oracle_f64_to_bf16.restype = C.c_uint16
        L.csl_oracle_e4m3_to_f64.argtypes = [C.c_uint8]
        L.csl_oracle_e4m3_to_f64.restype = dbl
        L.csl_oracle_f64_to_e4m3.argtypes = [dbl]
        L.csl_oracle_f64_to_e4m3.restype = C.c_uint8
        L.csl_oracle_e2m1_to_f64.argtypes = [C.c_int]
        L.csl_oracle_e2m1_to_f64.restype = dbl
        L.csl_oracle_f64_to_e2m1.argtypes = [dbl]
        L.csl_oracle_f64_to_e2m1.restype = C.c_int
        L.csl_oracle_mxfp4_block.argtypes = [vp, vp, vp]
        L.csl_oracle_mxfp4_block.restype = None
        L.csl_oracle_rope.argtypes = [vp, C.c_int, C.c_int, dbl, i64]
        L.csl_oracle_rope.restype = None
        L.csl_oracle_compress_insert.argtypes = [C.POINTER(Pool), vp, C.c_int, C.c_int, vp, vp, vp, vp, vp, dbl]
        L.csl_oracle_compress_insert.restype = C.c_int
        L.csl_oracle_index_topk.argtypes = [C.POINTER(Pool), vp, C.c_int, C.c_int, vp, vp, vp, vp, C.c_int,
                                            C.c_int, vp, vp, vp, i64]
        L.csl_oracle_index_topk.restype = C.c_int
        L.csl_oracle_hybrid_attn.argtypes = [C.POINTER(Pool), C.POINTER(Pool), vp, C.c_int, C.c_int, vp, vp,
                                             vp, C.c_int, vp, C.c_int, C.c_int, dbl, C.c_int, vp, vp, vp]
        L.csl_oracle_hybrid_attn.restype = C.c_int
        L.csl_oracle_q_norm_rope_insert.argtypes = [C.POINTER(Pool), vp, C.c_int, C.c_int, vp, vp, vp, vp, C.c_int,
                                                     vp, dbl, vp]
        L.csl_oracle_q_norm_rope_insert.restype = C.c_int
        L.csl_oracle_compress_rows.argtypes = [C.POINTER(Pool), C.c_int, vp, vp, vp, vp, dbl, vp]
        L.csl_oracle_compress_rows.restype = None
        L.csl_oracle_set_threads.argtypes = [C.c_int]
        L.csl_oracle_set_threads.restype = None
        L.csl_oracle_num_threads.argtypes = []
        L.csl_oracle_num_threads.restype = C.c_int
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous numpy arrays"
    return a.ctypes.data


def row_bytes(dim: int, dtype: int) -> int:
    return int(lib().csl_oracle_row_bytes(dim, dtype))


def bf16_to_f64(h: int) -> float:
    return float(lib().csl_oracle_bf16_to_f64(h))


def f64_to_bf16(v: float) -> int:
    return int(lib().csl_oracle_f64_to_bf16(v))


def e4m3_to_f64(c: int) -> float:
    return float(lib().csl_oracle_e4m3_to_f64(c))


def f64_to_e4m3(v: float) -> int:
    return int(lib().csl_oracle_f64_to_e4m3(v))


def e2m1_to_f64(c: int) -> float:
    return float(lib().csl_oracle_e2m1_to_f64(c))


def f64_to_e2m1(v: float) -> int:
    return int(lib().csl_oracle_f64_to_e2m1(v))


def mxfp4_block(y: np.ndarray) -> tuple:
    """One 32-element MXFP4 block of y: (16 code bytes, E8M0 scale code)."""
    yy = np.ascontiguousarray(y, dtype=np.float64)
    assert yy.shape == (32,)
    codes = np.zeros(16, np.uint8)
    sc = np.zeros(1, np.uint8)
    lib().csl_oracle_mxfp4_block(yy.ctypes.data, codes.ctypes.data, sc.ctypes.data)
    return codes, int(sc[0])


def rope(v: np.ndarray, rope_dims: int, theta: float, pos: int) -> np.ndarray:
    """RoPE of a copy of the fp64 vector v at integer position pos (negative = inverse)."""
    out = np.ascontiguousarray(v, dtype=np.float64).copy()
    lib().csl_oracle_rope(_p(out), out.shape[-1], rope_dims, float(theta), int(pos))
    return out


class HostPool:
    """A paged cache pool in host memory, same byte layout as the device pools."""

    def __init__(self, ratio, coff, dim, rope_dims, theta, dtype, num_pages, state=True, rows=None):
        self.ratio, self.coff, self.dim, self.rope_dims = ratio, coff, dim, rope_dims
        self.theta, self.dtype, self.num_pages = float(theta), dtype, num_pages
        self.row_bytes = row_bytes(dim, dtype)
        self.rows_per_page = BLOCK // ratio
        self.rows = rows if rows is not None else np.zeros((num_pages, self.rows_per_page, self.row_bytes), np.uint8)
        if state and ratio > 1:
            self.state_x = np.zeros((num_pages, BLOCK, dim), np.uint16)
            self.state_logits = np.zeros((num_pages, BLOCK, coff), np.float32)
        else:
            self.state_x = None
            self.state_logits = None

    def struct(self) -> Pool:
        return Pool(self.ratio, self.coff, self.dim, self.rope_dims, self.theta, self.dtype, self.num_pages,
                    _p(self.rows), _p(self.state_x), _p(self.state_logits))


def compress_insert(pool: HostPool, bt, start_pos, cu_new, x, logits=None, gain=None, eps=1e-6) -> int:
    bt = np.ascontiguousarray(bt, np.int32)
    st = np.ascontiguousarray(start_pos, np.int64)
    cu = np.ascontiguousarray(cu_new, np.int32)
    x = np.ascontiguousarray(x, np.uint16)
    lg = None if logits is None else np.ascontiguousarray(logits, np.float32)
    g = None if gain is None else np.ascontiguousarray(gain, np.float32)
    s = pool.struct()
    return lib().csl_oracle_compress_insert(C.byref(s), _p(bt), len(st), bt.shape[1], _p(st), _p(cu), _p(x),
                                            _p(lg), _p(g), float(eps))


def q_norm_rope_insert(pool: HostPool, bt, start_pos, cu_new, x, q, gain=None, eps=1e-6):
    """Query side of a step: every head of q [total][n_heads][dim] bf16 is
    RMS-normed (gain [dim] or None) and rotated at its token's position with
    the raw pool's RoPE; the raw rows RoPE(x_t, t) go into `pool` (ratio 1).
    Returns (q_out [total][n_heads][dim] uint16 bf16 bits, faults)."""
    bt = np.ascontiguousarray(bt, np.int32)
    st = np.ascontiguousarray(start_pos, np.int64)
    cu = np.ascontiguousarray(cu_new, np.int32)
    x = np.ascontiguousarray(x, np.uint16)
    q = np.ascontiguousarray(q, np.uint16)
    g = None if gain is None else np.ascontiguousarray(gain, np.float32)
    out = np.zeros_like(q)
    s = pool.struct()
    f = lib().csl_oracle_q_norm_rope_insert(C.byref(s), _p(bt), len(st), bt.shape[1], _p(st), _p(cu), _p(x), _p(q),
                                            q.shape[1], _p(g), float(eps), _p(out))
    return out, f


def compress_rows(ratio, coff, dim, rope_dims, theta, dtype, ids, x_win, logits_win=None, gain=None, eps=1e-6):
    """Stored rows of entries `ids` computed one by one from their windows:
    x_win [n][coff*ratio][dim] bf16 (tokens r(i+1)-W .. r(i+1)-1; rows at
    negative positions are ignored), logits_win [n][coff*ratio][coff] fp32
    (None for ratio 1).  Returns [n][row_bytes] uint8."""
    ids = np.ascontiguousarray(ids, np.int64)
    n = ids.shape[0]
    W = coff * ratio
    x_win = np.ascontiguousarray(x_win, np.uint16).reshape(n, W, dim)
    lg = None if logits_win is None else np.ascontiguousarray(logits_win, np.float32).reshape(n, W, coff)
    g = None if gain is None else np.ascontiguousarray(gain, np.float32)
    out = np.zeros((n, row_bytes(dim, dtype)), np.uint8)
    desc = Pool(ratio, coff, dim, rope_dims, float(theta), dtype, 0, None, None, None)
    lib().csl_oracle_compress_rows(C.byref(desc), n, _p(ids), _p(x_win), _p(lg), _p(g), float(eps), _p(out))
    return out


def index_topk(pool: HostPool, bt, q_seq, q_pos, q_idx, w, k, want_scores=False, max_cand=None):
    bt = np.ascontiguousarray(bt, np.int32)
    q_seq = np.ascontiguousarray(q_seq, np.int32)
    q_pos = np.ascontiguousarray(q_pos, np.int64)
    q_idx = np.ascontiguousarray(q_idx, np.uint16)
    w = np.ascontiguousarray(w, np.float32)
    nq, nh = w.shape
    topk = np.empty((nq, k), np.int32)
    kth = np.empty(nq, np.float64)
    scores = None
    if want_scores:
        if max_cand is None:
            max_cand = int(q_pos.max()) // pool.ratio if nq else 0
        scores = np.empty((nq, max(max_cand, 1)), np.float64)
    s = pool.struct()
    f = lib().csl_oracle_index_topk(C.byref(s), _p(bt), bt.shape[1], nq, _p(q_seq), _p(q_pos), _p(q_idx), _p(w),
                                    nh, k, _p(topk), _p(kth), _p(scores), int(max_cand or 0))
    return topk, kth, scores, f


def hybrid_attn(comp: HostPool | None, swa: HostPool, bt, q_seq, q_pos, q, topk=None, k=0, swa_window=128,
                softmax_scale=None, out_dtype=F32):
    """Returns (out, out_scales or None, out_f64, faults)."""
    bt = np.ascontiguousarray(bt, np.int32)
    q_seq = np.ascontiguousarray(q_seq, np.int32)
    q_pos = np.ascontiguousarray(q_pos, np.int64)
    q = np.ascontiguousarray(q, np.uint16)
    nq, nh, d = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(d)
    if topk is not None:
        topk = np.ascontiguousarray(topk, np.int32)
        k = topk.shape[1]
    if out_dtype == F32:
        out = np.empty((nq, nh, d), np.float32)
    elif out_dtype == BF16:
        out = np.empty((nq, nh, d), np.uint16)
    else:
        out = np.empty((nq, nh, d), np.uint8)
    scales = np.empty((nq, nh, d // 64), np.float32) if out_dtype == FP8 else None
    o64 = np.empty((nq, nh, d), np.float64)
    cs = comp.struct() if comp is not None else None
    ss = swa.struct()
    f = lib().csl_oracle_hybrid_attn(C.byref(cs) if cs is not None else None, C.byref(ss), _p(bt), bt.shape[1], nq,
                                     _p(q_seq), _p(q_pos), _p(q), nh, _p(topk), int(k), int(swa_window),
                                     float(softmax_scale), out_dtype, _p(out), _p(scales), _p(o64))
    return out, scales, o64, f


def set_threads(n: int) -> None:
    """Threads of the oracle's parallel loops (timing only)."""
    lib().csl_oracle_set_threads(int(n))


def num_threads() -> int:
    return int(lib().csl_oracle_num_threads())


def decode_rows(rows: np.ndarray, dim: int, dtype: int) -> np.ndarray:
    """fp64 values of stored rows [..., row_bytes] (bf16, fp8+scales or fp4+E8M0), via the oracle's own decoders."""
    shp = rows.shape[:-1]
    r = rows.reshape(-1, rows.shape[-1])
    out = np.empty((r.shape[0], dim), np.float64)
    if dtype == BF16:
        out[:] = bf16_array_to_f64(r.view(np.uint16)[:, :dim])
    elif dtype == FP8:
        table = np.array([e4m3_to_f64(c) for c in range(256)], np.float64)
        sc = r[:, dim:dim + 4 * (dim // 64)].copy().view(np.float32).astype(np.float64)
        out[:] = table[r[:, :dim]] * np.repeat(sc, 64, axis=1)
    elif dtype == FP4:
        table = np.array([e2m1_to_f64(c) for c in range(16)], np.float64)
        codes = np.empty((r.shape[0], dim), np.uint8)
        codes[:, 0::2] = r[:, :dim // 2] & 15
        codes[:, 1::2] = r[:, :dim // 2] >> 4
        sc = np.ldexp(1.0, r[:, dim // 2:dim // 2 + dim // 32].astype(np.int64) - 127)
        out[:] = table[codes] * np.repeat(sc, 32, axis=1)
    else:
        out[:] = r.view(np.float32)[:, :dim]
    return out.reshape(*shp, dim)


def bf16_array_to_f64(h: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp64: the pattern is the top half of an fp32."""
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

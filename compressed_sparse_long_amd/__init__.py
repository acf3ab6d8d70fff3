"""Python binding of libcsl.so, the gfx950 hybrid compressed-attention library.

Argument marshalling only: every step of the path runs in the library's HIP
kernels; torch supplies device memory and the stream.  The functions carry
the C ABI's names (include/csl.h) without the ``csl_`` prefix.  Importing this
module fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsl.so")

F32, BF16, FP8, FP4 = 0, 1, 2, 3
BLOCK = 256
KERNEL_COMPRESS, KERNEL_INDEX_SCORE, KERNEL_TOPK_SELECT, KERNEL_ATTN, KERNEL_ATTN_COMBINE, KERNEL_QSIDE = 0, 1, 2, 3, 4, 5
DEVERR_UNMAPPED_PAGE, DEVERR_TOPK_ID, DEVERR_POSITION, DEVERR_SEQ = 1, 2, 4, 8

_STATUS = {0: "CSL_OK", -1: "CSL_EINVAL", -2: "CSL_ERANGE", -3: "CSL_EALIGN", -4: "CSL_EWORKSPACE",
           -5: "CSL_EHIP", -6: "CSL_EUNSUPPORTED"}


class CslError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")


class _Pool(C.Structure):
    _fields_ = [
        ("ratio", C.c_int32), ("coff", C.c_int32), ("dim", C.c_int32), ("rope_dims", C.c_int32),
        ("rope_theta", C.c_double),
        ("dtype", C.c_int32), ("num_pages", C.c_int32),
        ("rows", C.c_void_p), ("state_x", C.c_void_p), ("state_logits", C.c_void_p),
    ]


class _InsertJob(C.Structure):
    _fields_ = [("pool", C.c_void_p), ("x", C.c_void_p), ("logits", C.c_void_p), ("gain", C.c_void_p)]


class _Pages(C.Structure):
    _fields_ = [("block_table", C.c_void_p), ("num_seqs", C.c_int32), ("max_blocks", C.c_int32)]


_lib = C.CDLL(LIB_PATH)
_vp, _i32, _i64, _sz, _f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t, C.c_float
_P = C.POINTER(_Pool)
_G = C.POINTER(_Pages)


def _sig(name, res, args):
    fn = getattr(_lib, name)
    fn.restype = res
    fn.argtypes = args
    return fn


_row_bytes = _sig("csl_row_bytes", _sz, [_i32, _i32])
_compress_insert = _sig("csl_compress_insert", C.c_int, [_P, _G, _vp, _vp, _i32, _vp, _vp, _vp, _f32, _vp])
_compress_insert_multi = _sig("csl_compress_insert_multi", C.c_int,
                              [_i32, C.POINTER(_InsertJob), _G, _vp, _vp, _i32, _f32, _vp])
_q_side = _sig("csl_q_norm_rope_insert", C.c_int, [_P, _G, _vp, _vp, _i32, _vp, _vp, _i32, _vp, _f32, _vp, _vp])
_index_topk_ws = _sig("csl_index_topk_workspace", _sz, [_i32, _i64, _i32])
_index_topk = _sig("csl_index_topk", C.c_int,
                   [_P, _G, _i32, _vp, _vp, _i64, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _sz, _vp])
class _QSideJob(C.Structure):
    _fields_ = [("swa", C.c_void_p), ("x", C.c_void_p), ("q", C.c_void_p), ("n_heads", C.c_int32),
                ("q_gain", C.c_void_p), ("q_out", C.c_void_p)]


_index_topk_insert = _sig("csl_index_topk_insert", C.c_int,
                          [_P, _G, _i32, _vp, _vp, _i64, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _sz, _i32,
                           C.POINTER(_InsertJob), _vp, _vp, _i32, _f32, C.POINTER(_QSideJob), _vp])
_attn_ws = _sig("csl_hybrid_attn_workspace", _sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i64])
_attn_decode = _sig("csl_hybrid_attn_decode", C.c_int,
                    [_P, _P, _G, _i32, _vp, _vp, _i64, _vp, _i32, _vp, _i32, _i32, _f32, _i32, _vp, _vp, _vp, _sz,
                     _vp])
_attn_decode_insert = _sig("csl_hybrid_attn_decode_insert", C.c_int,
                           [_P, _P, _G, _i32, _vp, _vp, _i64, _vp, _i32, _vp, _i32, _i32, _f32, _i32, _vp, _vp, _i32,
                            C.POINTER(_InsertJob), _vp, _vp, _i32, _f32, _vp, _sz, _vp])
_attn_prefill = _sig("csl_hybrid_attn_prefill", C.c_int,
                     [_P, _P, _G, _vp, _vp, _i32, _i64, _vp, _i32, _vp, _i32, _i32, _f32, _i32, _vp, _vp, _vp])
_fused_ws = _sig("csl_index_attn_decode_workspace", _sz, [_i32, _i32, _i64, _i32, _i32])
_fused = _sig("csl_index_attn_decode", C.c_int,
              [_P, _P, _P, _G, _i32, _vp, _vp, _i64, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _i32, _i32, _f32, _i32,
               _vp, _vp, _i32, C.POINTER(_InsertJob), _vp, _vp, _i32, _f32, C.POINTER(_QSideJob), _vp, _sz, _vp])
_fused_noalloc = _sig("csl_index_attn_decode_noalloc", C.c_int,
                      [_P, _P, _P, _G, _i32, _vp, _vp, _i64, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _i32, _i32, _f32,
                       _i32, _vp, _vp, _i32, C.POINTER(_InsertJob), _vp, _vp, _i32, _f32, C.POINTER(_QSideJob), _vp])
_last_error = _sig("csl_last_error", C.c_char_p, [])
_read_dev_err = _sig("csl_read_device_error", C.c_int, [C.POINTER(C.c_uint32)])
_timer_enable = _sig("csl_timer_enable", C.c_int, [_i32, _i32])
_timer_read = _sig("csl_timer_read", C.c_int, [_i32, C.POINTER(C.c_double), C.POINTER(C.c_int64)])

EXPORTS = ["csl_row_bytes", "csl_compress_insert", "csl_compress_insert_multi", "csl_q_norm_rope_insert",
           "csl_index_topk_workspace", "csl_index_topk", "csl_index_topk_insert",
           "csl_hybrid_attn_workspace", "csl_hybrid_attn_decode", "csl_hybrid_attn_decode_insert",
           "csl_hybrid_attn_prefill",
           "csl_index_attn_decode_workspace", "csl_index_attn_decode", "csl_index_attn_decode_noalloc",
           "csl_last_error",
           "csl_read_device_error", "csl_timer_enable", "csl_timer_read"]


def _check(st: int):
    if st != 0:
        raise CslError(st, _last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def row_bytes(dim: int, dtype: int) -> int:
    return int(_row_bytes(dim, dtype))


class Pool:
    """A paged pool: rows [num_pages][256/ratio][row_bytes] uint8, plus the compressor state
    (ratio > 1).  Tensors are supplied by the caller or allocated here with torch."""

    def __init__(self, ratio, coff, dim, rope_dims, theta, dtype, num_pages, device="cuda", state=True,
                 rows=None, state_x=None, state_logits=None):
        self.ratio, self.coff, self.dim, self.rope_dims = ratio, coff, dim, rope_dims
        self.theta, self.dtype, self.num_pages = float(theta), dtype, num_pages
        self.row_bytes = row_bytes(dim, dtype)
        self.rows_per_page = BLOCK // ratio
        if rows is None:
            rows = torch.zeros((num_pages, self.rows_per_page, self.row_bytes), dtype=torch.uint8, device=device)
        self.rows = rows
        if ratio > 1 and state and state_x is None:
            state_x = torch.zeros((num_pages, BLOCK, dim), dtype=torch.bfloat16, device=device)
            state_logits = torch.zeros((num_pages, BLOCK, coff), dtype=torch.float32, device=device)
        self.state_x, self.state_logits = state_x, state_logits

    def struct(self) -> _Pool:
        return _Pool(self.ratio, self.coff, self.dim, self.rope_dims, self.theta, self.dtype, self.num_pages,
                     _ptr(self.rows), _ptr(self.state_x), _ptr(self.state_logits))


def pages(block_table: torch.Tensor) -> _Pages:
    assert block_table.dtype == torch.int32 and block_table.is_contiguous()
    return _Pages(block_table.data_ptr(), block_table.shape[0], block_table.shape[1])


def compress_insert(pool: Pool, block_table, start_pos, cu_new, x, logits=None, gain=None, eps=1e-6, stream=None):
    ps = pool.struct()
    pg = pages(block_table)
    total = int(x.shape[0])
    _check(_compress_insert(C.byref(ps), C.byref(pg), _ptr(start_pos), _ptr(cu_new), total, _ptr(x), _ptr(logits),
                            _ptr(gain), float(eps), _stream(stream)))


def compress_insert_multi(jobs, block_table, start_pos, cu_new, eps=1e-6, stream=None):
    """jobs: list of (pool, x, logits or None, gain or None) sharing one batch of new tokens."""
    structs = [p.struct() for p, _, _, _ in jobs]
    arr = (_InsertJob * len(jobs))(*[_InsertJob(C.addressof(structs[i]), _ptr(x), _ptr(lg), _ptr(g))
                                     for i, (_, x, lg, g) in enumerate(jobs)])
    pg = pages(block_table)
    total = int(jobs[0][1].shape[0])
    _check(_compress_insert_multi(len(jobs), arr, C.byref(pg), _ptr(start_pos), _ptr(cu_new), total, float(eps),
                                  _stream(stream)))


def q_norm_rope_insert(swa: Pool, block_table, start_pos, cu_new, x, q, gain=None, eps=1e-6, q_out=None,
                       stream=None):
    """Per-head RMSNorm + RoPE of q [total][n_heads][dim] bf16 into q_out (default: in place) and the
    raw-key insert of x [total][dim] into `swa`, one launch.  Returns q_out."""
    q_out = q if q_out is None else q_out
    ps = swa.struct()
    pg = pages(block_table)
    _check(_q_side(C.byref(ps), C.byref(pg), _ptr(start_pos), _ptr(cu_new), int(q.shape[0]), _ptr(x), _ptr(q),
                   int(q.shape[1]), _ptr(gain), float(eps), _ptr(q_out), _stream(stream)))
    return q_out


def index_topk_workspace(num_q: int, max_q_pos: int, k: int) -> int:
    return int(_index_topk_ws(num_q, max_q_pos, k))


def index_topk(pool: Pool, block_table, q_seq, q_pos, max_q_pos, q_idx, w, k, topk, kth_score=None, ws=None,
               stream=None):
    ps = pool.struct()
    pg = pages(block_table)
    nq, nh = int(w.shape[0]), int(w.shape[1])
    _check(_index_topk(C.byref(ps), C.byref(pg), nq, _ptr(q_seq), _ptr(q_pos), int(max_q_pos), _ptr(q_idx), _ptr(w),
                       nh, int(k), _ptr(topk), _ptr(kth_score), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                       _stream(stream)))


def index_topk_insert(pool: Pool, block_table, q_seq, q_pos, max_q_pos, q_idx, w, k, topk, jobs, start_pos, cu_new,
                      kth_score=None, ws=None, eps=1e-6, qside=None, stream=None):
    """index_topk, then compress_insert_multi(jobs, ...), then (qside) q_norm_rope_insert on the same
    stream, the writes riding in the top-k launch.  jobs: list of (pool, x, logits or None, gain or
    None); qside: (swa pool, x, q, gain or None, q_out or None = in place)."""
    ps = pool.struct()
    pg = pages(block_table)
    nq, nh = int(w.shape[0]), int(w.shape[1])
    structs = [p.struct() for p, _, _, _ in jobs]
    arr = (_InsertJob * max(1, len(jobs)))(*[_InsertJob(C.addressof(structs[i]), _ptr(x), _ptr(lg), _ptr(g))
                                             for i, (_, x, lg, g) in enumerate(jobs)])
    qs, qsp = None, None
    if qside is not None:
        swa, qx, qq, qg, qo = qside
        qsp = swa.struct()
        qs = _QSideJob(C.addressof(qsp), _ptr(qx), _ptr(qq), int(qq.shape[1]), _ptr(qg), _ptr(qq if qo is None else qo))
    total = int(jobs[0][1].shape[0]) if jobs else int(qside[1].shape[0])
    _check(_index_topk_insert(C.byref(ps), C.byref(pg), nq, _ptr(q_seq), _ptr(q_pos), int(max_q_pos), _ptr(q_idx),
                              _ptr(w), nh, int(k), _ptr(topk), _ptr(kth_score), _ptr(ws),
                              0 if ws is None else ws.numel() * ws.element_size(), len(jobs), arr, _ptr(start_pos),
                              _ptr(cu_new), total, float(eps), None if qs is None else C.byref(qs), _stream(stream)))


def hybrid_attn_workspace(num_q, n_heads, dim, comp_ratio, k, swa_window, max_q_pos) -> int:
    return int(_attn_ws(num_q, n_heads, dim, comp_ratio, k, swa_window, max_q_pos))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zero-filled device workspace of at least `nbytes` (16-byte aligned): the
    decode calls keep arrival counters in its first 16 KiB, which must start at zero."""
    return torch.zeros(max(1, (int(nbytes) + 3) // 4), dtype=torch.float32, device=device)


def index_attn_decode_workspace(num_q: int, n_heads: int, max_q_pos: int, k: int, swa_window: int) -> int:
    return int(_fused_ws(num_q, n_heads, max_q_pos, k, swa_window))


def index_attn_decode(index_pool: Pool, comp: Pool, swa: Pool, block_table, q_seq, q_pos, max_q_pos, q_idx, w, k,
                      topk, q, swa_window, softmax_scale, out_dtype, out, out_scales=None, jobs=(), start_pos=None,
                      cu_new=None, kth_score=None, ws=None, eps=1e-6, qside=None, stream=None, noalloc=False):
    """index_topk_insert then hybrid_attn_decode in two launches (csl_index_attn_decode).  jobs and
    qside as in index_topk_insert; ws from workspace(index_attn_decode_workspace(...)).  noalloc=True
    calls csl_index_attn_decode_noalloc instead (no ws: the library's static scratch)."""
    ips, cs, ss = index_pool.struct(), comp.struct(), swa.struct()
    pg = pages(block_table)
    nq, nh = int(w.shape[0]), int(w.shape[1])
    jobs = list(jobs)
    structs = [p.struct() for p, _, _, _ in jobs]
    arr = (_InsertJob * max(1, len(jobs)))(*[_InsertJob(C.addressof(structs[i]), _ptr(x), _ptr(lg), _ptr(g))
                                             for i, (_, x, lg, g) in enumerate(jobs)])
    qs, qsp = None, None
    if qside is not None:
        qswa, qx, qq, qg, qo = qside
        qsp = qswa.struct()
        qs = _QSideJob(C.addressof(qsp), _ptr(qx), _ptr(qq), int(qq.shape[1]), _ptr(qg), _ptr(qq if qo is None else qo))
    total = int(jobs[0][1].shape[0]) if jobs else (int(qside[1].shape[0]) if qside is not None else 0)
    args = (C.byref(ips), C.byref(cs), C.byref(ss), C.byref(pg), nq, _ptr(q_seq), _ptr(q_pos), int(max_q_pos),
            _ptr(q_idx), _ptr(w), nh, int(k), _ptr(topk), _ptr(kth_score), _ptr(q), int(q.shape[1]),
            int(swa_window), float(softmax_scale), int(out_dtype), _ptr(out), _ptr(out_scales), len(jobs), arr,
            _ptr(start_pos), _ptr(cu_new), total, float(eps), None if qs is None else C.byref(qs))
    if noalloc:
        if ws is not None:
            raise ValueError("noalloc=True takes no ws")
        _check(_fused_noalloc(*args, _stream(stream)))
    else:
        _check(_fused(*args, _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def hybrid_attn_decode(comp: Pool | None, swa: Pool, block_table, q_seq, q_pos, max_q_pos, q, topk, k, swa_window,
                       softmax_scale, out_dtype, out, out_scales=None, ws=None, stream=None):
    cs = comp.struct() if comp is not None else None
    ss = swa.struct()
    pg = pages(block_table)
    nq, nh = int(q.shape[0]), int(q.shape[1])
    _check(_attn_decode(C.byref(cs) if cs is not None else None, C.byref(ss), C.byref(pg), nq, _ptr(q_seq),
                        _ptr(q_pos), int(max_q_pos), _ptr(q), nh, _ptr(topk), int(k), int(swa_window),
                        float(softmax_scale), int(out_dtype), _ptr(out), _ptr(out_scales), _ptr(ws),
                        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def hybrid_attn_decode_insert(comp: Pool | None, swa: Pool, block_table, q_seq, q_pos, max_q_pos, q, topk, k,
                              swa_window, softmax_scale, out_dtype, out, jobs, start_pos, cu_new, out_scales=None,
                              ws=None, eps=1e-6, stream=None):
    """compress_insert_multi(jobs, ...) and hybrid_attn_decode(...) with the inserts riding in the
    attention launch (csl_hybrid_attn_decode_insert); jobs as in compress_insert_multi."""
    cs = comp.struct() if comp is not None else None
    ss = swa.struct()
    pg = pages(block_table)
    nq, nh = int(q.shape[0]), int(q.shape[1])
    jobs = list(jobs)
    structs = [p.struct() for p, _, _, _ in jobs]
    arr = (_InsertJob * max(1, len(jobs)))(*[_InsertJob(C.addressof(structs[i]), _ptr(x), _ptr(lg), _ptr(g))
                                             for i, (_, x, lg, g) in enumerate(jobs)])
    total = int(jobs[0][1].shape[0]) if jobs else 0
    _check(_attn_decode_insert(C.byref(cs) if cs is not None else None, C.byref(ss), C.byref(pg), nq, _ptr(q_seq),
                               _ptr(q_pos), int(max_q_pos), _ptr(q), nh, _ptr(topk), int(k), int(swa_window),
                               float(softmax_scale), int(out_dtype), _ptr(out), _ptr(out_scales), len(jobs), arr,
                               _ptr(start_pos), _ptr(cu_new), total, float(eps), _ptr(ws),
                               0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def hybrid_attn_prefill(comp: Pool | None, swa: Pool, block_table, cu_q, q_pos_start, max_q_pos, q, topk, k,
                        swa_window, softmax_scale, out_dtype, out, out_scales=None, stream=None):
    cs = comp.struct() if comp is not None else None
    ss = swa.struct()
    pg = pages(block_table)
    nq, nh = int(q.shape[0]), int(q.shape[1])
    _check(_attn_prefill(C.byref(cs) if cs is not None else None, C.byref(ss), C.byref(pg), _ptr(cu_q),
                         _ptr(q_pos_start), nq, int(max_q_pos), _ptr(q), nh, _ptr(topk), int(k), int(swa_window),
                         float(softmax_scale), int(out_dtype), _ptr(out), _ptr(out_scales), _stream(stream)))


def read_device_error() -> int:
    v = C.c_uint32(0)
    _check(_read_dev_err(C.byref(v)))
    return int(v.value)


def timer_enable(kernel_id: int, on: bool = True):
    _check(_timer_enable(kernel_id, 1 if on else 0))


def timer_read(kernel_id: int):
    ms, n = C.c_double(0), C.c_int64(0)
    _check(_timer_read(kernel_id, C.byref(ms), C.byref(n)))
    return float(ms.value), int(n.value)


def last_error() -> str:
    return _last_error().decode()

"""Python binding of libmla_cc.so (MLA chunked-context prefill, MI355X / gfx950).

Argument marshalling only: every step of the path runs in the library's host
C++ and HIP kernels.  Function names and semantics are those of the C ABI in
``include/mla_cc.h``.  Device tensors are torch tensors (torch provides device
memory and streams); launches go on the current torch stream unless a stream
is given.  A missing library raises at import: there is no other code path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla_cc.so")

MLA_OK = 0
MLA_ERR_INVALID_ARG = 1
MLA_ERR_CAPACITY = 2
MLA_ERR_UNSUPPORTED = 3
MLA_ERR_HIP = 4
QK_HEAD_DIM = 192
V_HEAD_DIM = 128
NO_ALLOC_SCRATCH_BYTES = 128 << 20  # MLA_NO_ALLOC_SCRATCH_BYTES

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first (python mla_chunked_context_amd/build.py)")

_lib = ctypes.CDLL(LIB_PATH)

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_ptr = ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.c_void_p


class ChunkDesc(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "request_begin", "request_end", "token_begin", "token_end", "entry_begin", "num_entries",
        "num_rows", "max_seq_len", "max_query_len", "is_continuation")]


class ChunkedPrefillParams(ctypes.Structure):
    _fields_ = [
        ("q", _ptr), ("k_new", _ptr), ("v_new", _ptr), ("k_cache", _ptr), ("v_cache", _ptr),
        ("block_table", _ptr), ("num_blocks", _i64), ("block_size", _i32), ("block_table_width", _i32),
        ("context_lens", _ptr), ("query_lens", _ptr), ("num_requests", _i32), ("num_heads", _i32),
        ("scale", ctypes.c_float), ("workspace_rows", _i64), ("max_context_chunk", _i64),
        ("split_alignment", _i32), ("out", _ptr), ("out_lse", _ptr), ("scratch", _ptr), ("scratch_bytes", _i64),
    ]


class DcpRanks(ctypes.Structure):
    _fields_ = [
        ("world_size", _i32), ("interleave", _i32), ("k_cache", ctypes.POINTER(_ptr)),
        ("v_cache", ctypes.POINTER(_ptr)), ("block_table", ctypes.POINTER(_ptr)), ("num_blocks", _i64p),
        ("block_table_width", _i32p),
    ]


def _sig(name, *argtypes):
    try:
        f = getattr(_lib, name)
    except AttributeError as e:
        raise ImportError(f"{LIB_PATH} does not export {name}: it is stale, rebuild it") from e
    f.argtypes = list(argtypes)
    f.restype = ctypes.c_int
    return f


_lib.mla_status_string.argtypes = [ctypes.c_int]
_lib.mla_status_string.restype = ctypes.c_char_p
_lib.mla_abi_version.argtypes = []
_lib.mla_abi_version.restype = ctypes.c_int
_plan = _sig("mla_plan_context_chunks", _i32p, _i32p, _i32, _i64, _i64, _i32, ctypes.POINTER(ChunkDesc), _i32,
             _i32p, _i32p, _i32p, _i32, _i32p)
_token_info = _sig("mla_prefill_token_info", _i32p, _i32p, _i32, _i64p, _i32p, _i32, _i32p)
_init = _sig("mla_init_context_partial", _ptr, _ptr, _i64, _i64, _i64, _i32, _i32, _ptr)
_gather = _sig("mla_gather_context", _ptr, _ptr, _i64, _i32, _i32, _ptr, _i32, _ptr, _ptr, _ptr, _i32, _i32,
               _ptr, _ptr, _ptr)
_chunk_attn = _sig("mla_context_chunk_attn", _ptr, _ptr, _ptr, _ptr, _ptr, _i32, _i32, _i32, ctypes.c_float,
                   _ptr, _ptr, _i64, _ptr)
_suffix_attn = _sig("mla_causal_suffix_attn", _ptr, _ptr, _ptr, _ptr, _i32, _i32, _i32, ctypes.c_float, _ptr,
                    _ptr, _i64, _ptr)
_merge = _sig("mla_merge_attn_states", _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _i64, _i32, _i32, _i64, _i64, _i64,
              _i64, _ptr)
_mask = _sig("mla_mask_empty_context", _ptr, _i64, _ptr, _i32, _ptr, _ptr, _i32, _i64, _i32, _i32, _ptr)
_scratch_size = _sig("mla_chunked_prefill_scratch_size", ctypes.POINTER(ChunkedPrefillParams), _i64p)
_prefill = _sig("mla_chunked_prefill", ctypes.POINTER(ChunkedPrefillParams), _ptr)
_prefill_no_alloc = _sig("mla_chunked_prefill_no_alloc", ctypes.POINTER(ChunkedPrefillParams), _ptr)
_plan_dcp = _sig("mla_plan_dcp_context_chunks", _i32p, _i32p, _i32, _i64, _i64, _i32, _i32, _i32,
                 ctypes.POINTER(ChunkDesc), _i32, _i32p, _i32p, _i32p, _i32p, _i32p, _i32, _i32p)
_dcp_reorg = _sig("mla_dcp_reorganize_context", _ptr, _ptr, _i32, _i32, _i32, _i32, _ptr, _ptr, _ptr, _i32, _i32,
                  _ptr, _ptr, _ptr)
_dcp_scratch_size = _sig("mla_dcp_chunked_prefill_scratch_size", ctypes.POINTER(ChunkedPrefillParams),
                         ctypes.POINTER(DcpRanks), _i64p)
_dcp_prefill = _sig("mla_dcp_chunked_prefill", ctypes.POINTER(ChunkedPrefillParams), ctypes.POINTER(DcpRanks), _ptr)
_plan_windows = _sig("mla_plan_uniform_windows", _i32p, _i32, _i64, _i32, _i64p, _i32p)
_uw_scratch_size = _sig("mla_uniform_window_prefill_scratch_size", ctypes.POINTER(ChunkedPrefillParams), _i64p)
_uw_prefill = _sig("mla_uniform_window_prefill", ctypes.POINTER(ChunkedPrefillParams), _ptr)

class KernelTime(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


KERNEL_KINDS = ["init", "gather", "chunk_attn", "suffix_attn", "merge", "mask", "dcp_reorg"]
_timing_enable = _sig("mla_kernel_timing_enable", ctypes.c_int)
_timing_read = _sig("mla_kernel_timing_read", ctypes.POINTER(KernelTime))

EXPORTED = [
    "mla_status_string", "mla_abi_version", "mla_plan_context_chunks", "mla_prefill_token_info",
    "mla_init_context_partial", "mla_gather_context", "mla_context_chunk_attn", "mla_causal_suffix_attn",
    "mla_merge_attn_states", "mla_chunked_prefill_scratch_size", "mla_chunked_prefill", "mla_chunked_prefill_no_alloc",
    "mla_kernel_timing_enable", "mla_kernel_timing_read", "mla_mask_empty_context", "mla_plan_uniform_windows",
    "mla_uniform_window_prefill_scratch_size", "mla_uniform_window_prefill", "mla_plan_dcp_context_chunks",
    "mla_dcp_reorganize_context", "mla_dcp_chunked_prefill_scratch_size", "mla_dcp_chunked_prefill",
]


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {mla_status_string(status)} (status {status})")


def _check(status: int, where: str):
    if status != MLA_OK:
        raise MlaError(status, where)


def mla_status_string(status: int) -> str:
    return _lib.mla_status_string(status).decode()


def mla_abi_version() -> int:
    return _lib.mla_abi_version()


def _i32_array(x):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    return a, a.ctypes.data_as(_i32p)


# ------------------------------------------------------------------ host


def mla_plan_context_chunks(context_lens, query_lens, row_budget, max_context_chunk=0, split_alignment=64):
    """Returns (chunks: list of dict, entry_starts int32[E], entry_seq_lens int32[E])."""
    ctx, ctx_p = _i32_array(context_lens)
    ql, ql_p = _i32_array(query_lens)
    n = len(ctx)
    if len(ql) != n:
        raise ValueError("context_lens and query_lens differ in length")
    nc, ne = _i32(0), _i32(0)
    st = _plan(ctx_p, ql_p, n, row_budget, max_context_chunk, split_alignment, None, 0, ctypes.byref(nc), None,
               None, 0, ctypes.byref(ne))
    if st not in (MLA_OK, MLA_ERR_CAPACITY):
        _check(st, "mla_plan_context_chunks")
    chunks = (ChunkDesc * max(1, nc.value))()
    starts = np.zeros(max(1, ne.value), dtype=np.int32)
    lens = np.zeros(max(1, ne.value), dtype=np.int32)
    _check(_plan(ctx_p, ql_p, n, row_budget, max_context_chunk, split_alignment, chunks, nc.value,
                 ctypes.byref(nc), starts.ctypes.data_as(_i32p), lens.ctypes.data_as(_i32p), ne.value,
                 ctypes.byref(ne)), "mla_plan_context_chunks")
    out = [{f: getattr(chunks[i], f) for f, _ in ChunkDesc._fields_} for i in range(nc.value)]
    return out, starts[:ne.value].copy(), lens[:ne.value].copy()


def mla_prefill_token_info(context_lens, query_lens):
    """Returns (prefix_num_tokens, [(begin, end), ...] of requests without context)."""
    ctx, ctx_p = _i32_array(context_lens)
    ql, ql_p = _i32_array(query_lens)
    pnt, ne = _i64(0), _i32(0)
    st = _token_info(ctx_p, ql_p, len(ctx), ctypes.byref(pnt), None, 0, ctypes.byref(ne))
    if st not in (MLA_OK, MLA_ERR_CAPACITY):
        _check(st, "mla_prefill_token_info")
    sl = np.zeros(2 * max(1, ne.value), dtype=np.int32)
    _check(_token_info(ctx_p, ql_p, len(ctx), ctypes.byref(pnt), sl.ctypes.data_as(_i32p), ne.value,
                       ctypes.byref(ne)), "mla_prefill_token_info")
    return pnt.value, [(int(sl[2 * i]), int(sl[2 * i + 1])) for i in range(ne.value)]


def mla_plan_dcp_context_chunks(context_lens, query_lens, row_budget, world_size, interleave=1,
                                max_context_chunk=0, split_alignment=64):
    """Returns (chunks, entry_starts, entry_seq_lens, entry_local_starts, entry_local_lens)."""
    ctx, ctx_p = _i32_array(context_lens)
    ql, ql_p = _i32_array(query_lens)
    n = len(ctx)
    if len(ql) != n:
        raise ValueError("context_lens and query_lens differ in length")
    nc, ne = _i32(0), _i32(0)
    args = (ctx_p, ql_p, n, row_budget, max_context_chunk, split_alignment, world_size, interleave)
    st = _plan_dcp(*args, None, 0, ctypes.byref(nc), None, None, None, None, 0, ctypes.byref(ne))
    if st not in (MLA_OK, MLA_ERR_CAPACITY):
        _check(st, "mla_plan_dcp_context_chunks")
    chunks = (ChunkDesc * max(1, nc.value))()
    arrs = [np.zeros(max(1, ne.value), dtype=np.int32) for _ in range(4)]
    _check(_plan_dcp(*args, chunks, nc.value, ctypes.byref(nc), *[a.ctypes.data_as(_i32p) for a in arrs], ne.value,
                     ctypes.byref(ne)), "mla_plan_dcp_context_chunks")
    out = [{f: getattr(chunks[i], f) for f, _ in ChunkDesc._fields_} for i in range(nc.value)]
    return (out, *[a[:ne.value].copy() for a in arrs])


def mla_plan_uniform_windows(context_lens, workspace_rows, split_alignment=64):
    """Returns (window, num_iterations) of the uniform-window scheduler."""
    ctx, ctx_p = _i32_array(context_lens)
    w, it = _i64(0), _i32(0)
    _check(_plan_windows(ctx_p, len(ctx), workspace_rows, split_alignment, ctypes.byref(w), ctypes.byref(it)),
           "mla_plan_uniform_windows")
    return w.value, it.value


# ---------------------------------------------------------------- device


def _dptr(t):
    """Device pointer of a torch tensor (or None -> NULL)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmla_cc must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def mla_init_context_partial(out, lse, row_begin, row_end, stream=None):
    """out [T, H, D] bf16, lse [H, stride] fp32."""
    T, H, D = out.shape
    _check(_init(_dptr(out), _dptr(lse), lse.shape[1], row_begin, row_end, H, D, _stream(stream)),
           "mla_init_context_partial")


def mla_gather_context(k_cache, v_cache, block_table, entry_request, entry_starts, entry_row_offsets, num_rows,
                       ws_k, ws_v, stream=None):
    nb, bs, H, _ = k_cache.shape
    _check(_gather(_dptr(k_cache), _dptr(v_cache), nb, bs, H, _dptr(block_table), block_table.shape[1],
                   _dptr(entry_request), _dptr(entry_starts), _dptr(entry_row_offsets), entry_request.numel(),
                   num_rows, _dptr(ws_k), _dptr(ws_v), _stream(stream)), "mla_gather_context")


def mla_context_chunk_attn(q, k, v, cu_q, cu_k, max_q, scale, out, lse, stream=None):
    """q [Tq, H, 192], k [Tk, H, 192], v [Tk, H, 128]; cu_q/cu_k int32 [n+1] on device;
    out [Tq, H, 128] bf16; lse [H, stride] fp32."""
    _check(_chunk_attn(_dptr(q), _dptr(k), _dptr(v), _dptr(cu_q), _dptr(cu_k), cu_q.numel() - 1, max_q,
                       q.shape[1], scale, _dptr(out), _dptr(lse), lse.shape[1], _stream(stream)),
           "mla_context_chunk_attn")


def mla_causal_suffix_attn(q, k_new, v_new, cu_q, max_q, scale, out, lse, stream=None):
    _check(_suffix_attn(_dptr(q), _dptr(k_new), _dptr(v_new), _dptr(cu_q), cu_q.numel() - 1, max_q, q.shape[1],
                        scale, _dptr(out), _dptr(lse), lse.shape[1], _stream(stream)), "mla_causal_suffix_attn")


def mla_merge_attn_states(out, out_lse, prefix_out, prefix_lse, suffix_out, suffix_lse, prefix_num_tokens=None,
                          stream=None):
    """out/prefix_out/suffix_out [T, H, D] bf16; LSEs [H, stride] fp32 (out_lse may be None)."""
    T, H, D = suffix_out.shape
    pnt = T if prefix_num_tokens is None else prefix_num_tokens
    _check(_merge(_dptr(out), _dptr(out_lse), _dptr(prefix_out), _dptr(prefix_lse), _dptr(suffix_out),
                  _dptr(suffix_lse), T, H, D, out_lse.shape[1] if out_lse is not None else 0,
                  prefix_lse.shape[1] if prefix_lse is not None else 0, suffix_lse.shape[1], pnt,
                  _stream(stream)), "mla_merge_attn_states")


def mla_mask_empty_context(lse, output, query_start_loc, context_start_loc, stream=None):
    """In place.  lse [H, stride] fp32; output [T, H, D] bf16 or fp32; start locs int32 [N+1] on device."""
    T, H, D = output.shape
    _check(_mask(_dptr(lse), lse.shape[1], _dptr(output), output.element_size(), _dptr(query_start_loc),
                 _dptr(context_start_loc), query_start_loc.numel() - 1, T, H, D, _stream(stream)),
           "mla_mask_empty_context")


def make_prefill_params(q, k_new, v_new, k_cache, v_cache, block_table, context_lens, query_lens, workspace_rows,
                        split_alignment, scale, out=None, out_lse=None, scratch=None, max_context_chunk=0):
    """Fill a ChunkedPrefillParams.  The returned object keeps the host lens alive."""
    ctx, _ = _i32_array(context_lens)
    ql, _ = _i32_array(query_lens)
    p = ChunkedPrefillParams()
    p.q, p.k_new, p.v_new = _dptr(q), _dptr(k_new), _dptr(v_new)
    p.k_cache, p.v_cache, p.block_table = _dptr(k_cache), _dptr(v_cache), _dptr(block_table)
    p.num_blocks = k_cache.shape[0] if k_cache is not None else 0
    p.block_size = k_cache.shape[1] if k_cache is not None else 1
    p.block_table_width = block_table.shape[1] if block_table is not None else 0
    p.context_lens = ctx.ctypes.data
    p.query_lens = ql.ctypes.data
    p.num_requests = len(ctx)
    p.num_heads = q.shape[1]
    p.scale = scale
    p.workspace_rows = workspace_rows
    p.max_context_chunk = max_context_chunk
    p.split_alignment = split_alignment
    p.out = _dptr(out)
    p.out_lse = _dptr(out_lse)
    p.scratch = _dptr(scratch)
    p.scratch_bytes = scratch.numel() * scratch.element_size() if scratch is not None else 0
    p._keep = (ctx, ql)
    return p


def mla_chunked_prefill_scratch_size(params: ChunkedPrefillParams) -> int:
    n = _i64(0)
    _check(_scratch_size(ctypes.byref(params), ctypes.byref(n)), "mla_chunked_prefill_scratch_size")
    return n.value


def mla_chunked_prefill(params: ChunkedPrefillParams, stream=None):
    _check(_prefill(ctypes.byref(params), _stream(stream)), "mla_chunked_prefill")


def mla_chunked_prefill_no_alloc(params: ChunkedPrefillParams, stream=None):
    """params.scratch is not read: the library's own device buffer is used."""
    _check(_prefill_no_alloc(ctypes.byref(params), _stream(stream)), "mla_chunked_prefill_no_alloc")


def mla_dcp_reorganize_context(gathered_k, gathered_v, world_size, interleave, local_rows, entry_starts,
                               entry_row_offsets, entry_local_offsets, num_rows, ws_k, ws_v, stream=None):
    """Device tensors; entry arrays int32 on the device."""
    _check(_dcp_reorg(_dptr(gathered_k), _dptr(gathered_v), gathered_k.shape[1], world_size, interleave, local_rows,
                      _dptr(entry_starts), _dptr(entry_row_offsets), _dptr(entry_local_offsets),
                      entry_starts.numel(), num_rows, _dptr(ws_k), _dptr(ws_v), _stream(stream)),
           "mla_dcp_reorganize_context")


def make_dcp_ranks(rank_caches, interleave=1):
    """DcpRanks over a list of per-rank caches (objects with k_cache, v_cache,
    block_table tensors).  The returned struct keeps its host arrays alive."""
    D = len(rank_caches)
    r = DcpRanks()
    r.world_size, r.interleave = D, interleave
    r._k = (_ptr * D)(*[_dptr(x.k_cache) for x in rank_caches])
    r._v = (_ptr * D)(*[_dptr(x.v_cache) for x in rank_caches])
    r._t = (_ptr * D)(*[_dptr(x.block_table) for x in rank_caches])
    r._nb = (_i64 * D)(*[x.k_cache.shape[0] for x in rank_caches])
    r._w = (_i32 * D)(*[x.block_table.shape[1] for x in rank_caches])
    r.k_cache, r.v_cache, r.block_table = r._k, r._v, r._t
    r.num_blocks = ctypes.cast(r._nb, _i64p)
    r.block_table_width = ctypes.cast(r._w, _i32p)
    return r


def mla_dcp_chunked_prefill_scratch_size(params: ChunkedPrefillParams, ranks: DcpRanks) -> int:
    n = _i64(0)
    _check(_dcp_scratch_size(ctypes.byref(params), ctypes.byref(ranks), ctypes.byref(n)),
           "mla_dcp_chunked_prefill_scratch_size")
    return n.value


def mla_dcp_chunked_prefill(params: ChunkedPrefillParams, ranks: DcpRanks, stream=None):
    _check(_dcp_prefill(ctypes.byref(params), ctypes.byref(ranks), _stream(stream)), "mla_dcp_chunked_prefill")


def mla_uniform_window_prefill_scratch_size(params: ChunkedPrefillParams) -> int:
    n = _i64(0)
    _check(_uw_scratch_size(ctypes.byref(params), ctypes.byref(n)), "mla_uniform_window_prefill_scratch_size")
    return n.value


def mla_uniform_window_prefill(params: ChunkedPrefillParams, stream=None):
    _check(_uw_prefill(ctypes.byref(params), _stream(stream)), "mla_uniform_window_prefill")


def mla_kernel_timing_enable(enable: bool = True):
    _check(_timing_enable(1 if enable else 0), "mla_kernel_timing_enable")


def mla_kernel_timing_read():
    """{kind: (launches, total_ms)} of the launches timed since the last read."""
    arr = (KernelTime * len(KERNEL_KINDS))()
    _check(_timing_read(arr), "mla_kernel_timing_read")
    return {k: (arr[i].launches, arr[i].total_ms) for i, k in enumerate(KERNEL_KINDS)}

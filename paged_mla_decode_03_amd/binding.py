"""Thin ctypes binding over the C ABI in include/mla_decode.h.

Argument marshalling only: every step of the decode runs in the HIP library.
torch supplies device memory and the current HIP stream.  Nothing here falls
back to a CPU path: if the library is missing, every call raises.

Interface modelled on FlashInfer's paged MLA decode API (docs page
"flashinfer.attention.prims_ts.prims_ts_batch_decode_with_kv_cache_mla",
signature and contract): fixed [B, SQ, H, 576] or packed [total_q, H, 576]
queries with qo_indptr, a [pages, page_size, 576] (or [pages, 1, page_size, 576])
cache, block_tables / seq_lens, caller-owned workspace, optional preallocated
output, bmm1/bmm2 scales and a causal or dense mask.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla_decode.so")

MLA_OK = 0
MLA_KV_BF16 = 0
MLA_KV_FP8_E4M3FN = 1
KV_LORA_RANK = 512
QK_ROPE_HEAD_DIM = 64
D_QK = KV_LORA_RANK + QK_ROPE_HEAD_DIM


class MlaOptions(ctypes.Structure):
    _fields_ = [
        ("bmm1_scale", ctypes.c_void_p),
        ("bmm2_scale", ctypes.c_void_p),
        ("sinks", ctypes.c_void_p),
        ("seq_lens_global", ctypes.c_void_p),
        ("cp_world", ctypes.c_int32),
        ("cp_rank", ctypes.c_int32),
        ("sparse_top_k", ctypes.c_int32),
        ("q_fp8", ctypes.c_int32),
    ]


class MlaDims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("q_len_fixed", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("block_table_stride", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("kv_lora_rank", ctypes.c_int32),
        ("qk_rope_head_dim", ctypes.c_int32),
    ]


_lib = None


def load_library():
    """Load the HIP library once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} missing (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.mla_decode_paged.argtypes = [vp, vp, vp, vp, vp, i32, i32, f32, f32, ctypes.c_int, vp, vp, vp, sz,
                                     ctypes.POINTER(MlaDims), vp]
    lib.mla_decode_paged.restype = ctypes.c_int
    lib.mla_decode_paged_ex.argtypes = [vp, vp, vp, vp, vp, i32, i32, f32, f32, ctypes.c_int, vp, vp, vp, sz,
                                        ctypes.POINTER(MlaDims), vp, ctypes.POINTER(MlaOptions)]
    lib.mla_decode_paged_ex.restype = ctypes.c_int
    lib.mla_decode_paged_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, f32, f32, ctypes.c_int, vp, vp,
                                             ctypes.POINTER(MlaDims), vp]
    lib.mla_decode_paged_noalloc.restype = ctypes.c_int
    lib.mla_merge_partials.argtypes = [vp, vp, i32, i64, vp, vp, vp]
    lib.mla_merge_partials.restype = ctypes.c_int
    lib.mla_decode_check_contract.argtypes = [vp, vp, vp, i32, i32, ctypes.c_int, ctypes.POINTER(MlaDims), vp, vp]
    lib.mla_decode_check_contract.restype = ctypes.c_int
    lib.mla_decode_paged_workspace_size.argtypes = [ctypes.POINTER(MlaDims), i32, i32, ctypes.c_int]
    lib.mla_decode_paged_workspace_size.restype = sz
    lib.mla_decode_paged_ex_workspace_size.argtypes = [ctypes.POINTER(MlaDims), i32, i32, ctypes.c_int,
                                                       ctypes.POINTER(MlaOptions)]
    lib.mla_decode_paged_ex_workspace_size.restype = sz
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_decode_internal_set_grid_override.argtypes = [i32]
    lib.mla_decode_internal_set_grid_override.restype = None
    lib.mla_decode_internal_set_segment_cost.argtypes = [i32]
    lib.mla_decode_internal_set_segment_cost.restype = None
    lib.mla_decode_internal_set_work_groups.argtypes = [i32]
    lib.mla_decode_internal_set_work_groups.restype = None
    lib.mla_decode_internal_set_kernel_events.argtypes = [vp, vp, vp]
    lib.mla_decode_internal_set_kernel_events.restype = None
    lib.mla_decode_internal_fp8_to_bf16.argtypes = [vp, vp, i64, vp]
    lib.mla_decode_internal_fp8_to_bf16.restype = ctypes.c_int
    _lib = lib
    return lib


def mla_status_string(status):
    return load_library().mla_status_string(int(status)).decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def make_dims(*, batch, num_heads, q_len_fixed, total_q, page_size, num_pages, block_table_stride, kv_dtype,
              kv_lora_rank=KV_LORA_RANK, qk_rope_head_dim=QK_ROPE_HEAD_DIM):
    return MlaDims(batch, num_heads, q_len_fixed, total_q, page_size, num_pages, block_table_stride, kv_dtype,
                   kv_lora_rank, qk_rope_head_dim)


def mla_decode_paged_workspace_size(dims, max_seq_len, max_q_len, want_lse=False):
    return int(load_library().mla_decode_paged_workspace_size(ctypes.byref(dims), int(max_seq_len),
                                                             int(max_q_len), int(bool(want_lse))))


def mla_decode_paged_ex_workspace_size(dims, max_seq_len, max_q_len, want_lse, opts):
    return int(load_library().mla_decode_paged_ex_workspace_size(
        ctypes.byref(dims), int(max_seq_len), int(max_q_len), int(bool(want_lse)),
        None if opts is None else ctypes.byref(opts)))


def mla_decode_paged(q, kv_cache, block_tables, seq_lens, qo_indptr, max_seq_len, max_q_len, bmm1_scale,
                     bmm2_scale, causal, out, lse, workspace, workspace_bytes, dims, stream=None):
    """Direct call of the C entry point (tensors or raw device pointers). Returns the status."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    return int(load_library().mla_decode_paged(
        _ptr(q), _ptr(kv_cache), _ptr(block_tables), _ptr(seq_lens), _ptr(qo_indptr), int(max_seq_len),
        int(max_q_len), float(bmm1_scale), float(bmm2_scale), int(bool(causal)), _ptr(out), _ptr(lse),
        _ptr(workspace), int(workspace_bytes), ctypes.byref(dims), stream))


NOALLOC_SCRATCH_BYTES = 64 << 20  # MLA_NOALLOC_SCRATCH_BYTES in include/mla_decode.h


def mla_decode_paged_noalloc(q, kv_cache, block_tables, seq_lens, qo_indptr, max_seq_len, max_q_len, bmm1_scale,
                             bmm2_scale, causal, out, lse, dims, stream=None):
    """Direct call of the no-allocation C entry point (the library's own
    per-device workspace).  Returns the status."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    return int(load_library().mla_decode_paged_noalloc(
        _ptr(q), _ptr(kv_cache), _ptr(block_tables), _ptr(seq_lens), _ptr(qo_indptr), int(max_seq_len),
        int(max_q_len), float(bmm1_scale), float(bmm2_scale), int(bool(causal)), _ptr(out), _ptr(lse),
        ctypes.byref(dims), stream))


def mla_decode_paged_ex(q, kv_cache, block_tables, seq_lens, qo_indptr, max_seq_len, max_q_len, bmm1_scale,
                        bmm2_scale, causal, out, lse, workspace, workspace_bytes, dims, opts, stream=None):
    """Direct call of the C entry point with device-resident options (an
    MlaOptions or None).  Returns the status."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    return int(load_library().mla_decode_paged_ex(
        _ptr(q), _ptr(kv_cache), _ptr(block_tables), _ptr(seq_lens), _ptr(qo_indptr), int(max_seq_len),
        int(max_q_len), float(bmm1_scale), float(bmm2_scale), int(bool(causal)), _ptr(out), _ptr(lse),
        _ptr(workspace), int(workspace_bytes), ctypes.byref(dims), stream,
        None if opts is None else ctypes.byref(opts)))


def set_grid_override(grid):
    """Test hook: force the persistent grid size (0 = one workgroup per CU)."""
    load_library().mla_decode_internal_set_grid_override(int(grid))


def set_segment_cost(tiles):
    """Tuning hook: the work split's cost of a segment start, in tiles
    (negative restores the default)."""
    load_library().mla_decode_internal_set_segment_cost(int(tiles))


def set_work_groups(enable):
    """Tuning hook: let launches whose requests all hold the same 2, 4 or 8
    units walk each request's tiles with a group of workgroups (True, the
    default; decided on the device), or always split unit by unit (False)."""
    load_library().mla_decode_internal_set_work_groups(int(bool(enable)))


def set_kernel_events(start_event, stop_event, decode_event=None):
    """Measurement hook: record torch.cuda.Event (HIP events) on the launch
    stream of every later call: start_event before its first kernel,
    stop_event after its last, decode_event (optional) right after the decode
    kernel.  set_kernel_events(None, None) turns it off.  torch only counts an
    event as recorded once torch itself has recorded it, so record each event
    once through torch before handing it over."""
    lib = load_library()
    if start_event is None or stop_event is None:
        lib.mla_decode_internal_set_kernel_events(None, None, None)
    else:
        lib.mla_decode_internal_set_kernel_events(start_event.cuda_event,
                                                  None if decode_event is None else decode_event.cuda_event,
                                                  stop_event.cuda_event)


def fp8_to_bf16_device(codes):
    """Test hook: widen a uint8 device tensor of fp8 E4M3FN codes (length a
    multiple of 8) to bf16 with the kernel's own conversion."""
    assert codes.dtype == torch.uint8 and codes.is_cuda and codes.numel() % 8 == 0
    out = torch.empty(codes.numel(), dtype=torch.bfloat16, device=codes.device)
    rc = load_library().mla_decode_internal_fp8_to_bf16(codes.data_ptr(), out.data_ptr(), codes.numel() // 8,
                                                       torch.cuda.current_stream().cuda_stream)
    if rc != MLA_OK:
        raise RuntimeError(mla_status_string(rc))
    return out


def _kv_code(dtype):
    if dtype == torch.bfloat16:
        return MLA_KV_BF16
    if dtype == torch.float8_e4m3fn:
        return MLA_KV_FP8_E4M3FN
    raise TypeError(f"kv_cache dtype {dtype} not supported (bf16 or float8_e4m3fn)")


def dims_for(query, kv_cache, block_tables, seq_lens, qo_indptr, max_seq_len_q):
    if kv_cache.dim() == 4:
        if kv_cache.shape[1] != 1:
            raise ValueError("rank-4 kv_cache must be [pages, 1, page_size, 576]")
        kv_cache = kv_cache.squeeze(1)
    if kv_cache.dim() != 3 or kv_cache.shape[-1] != D_QK:
        raise ValueError("kv_cache must be [pages, page_size, 576]")
    if query.shape[-1] != D_QK:
        raise ValueError(f"query rows must be {D_QK} wide (512 latent + 64 RoPE), got {query.shape[-1]}")
    if seq_lens.dim() != 1:
        raise ValueError("seq_lens must be 1-D [B]")
    B = int(seq_lens.shape[0])
    if block_tables.dim() != 2 or int(block_tables.shape[0]) != B:
        raise ValueError(f"block_tables must be 2-D [B={B}, W]")
    if qo_indptr is not None and (qo_indptr.dim() != 1 or int(qo_indptr.shape[0]) != B + 1
                                  or not qo_indptr.is_contiguous()):
        raise ValueError(f"qo_indptr must be a contiguous 1-D tensor of B+1={B + 1} offsets")
    if qo_indptr is None:
        if query.dim() != 4 or query.shape[0] != B:
            raise ValueError("fixed launch needs query [B, SQ, H, 576]")
        sq, H = int(query.shape[1]), int(query.shape[2])
        total_q = B * sq
        max_q = sq
    else:
        if query.dim() != 3:
            raise ValueError("packed launch needs query [total_q, H, 576]")
        if max_seq_len_q is None:
            raise ValueError("max_seq_len_q is required with qo_indptr")
        total_q, H = int(query.shape[0]), int(query.shape[1])
        sq = int(max_seq_len_q)
        max_q = int(max_seq_len_q)
    dims = make_dims(batch=B, num_heads=H, q_len_fixed=sq, total_q=total_q, page_size=int(kv_cache.shape[1]),
                     num_pages=int(kv_cache.shape[0]), block_table_stride=int(block_tables.shape[1]),
                     kv_dtype=_kv_code(kv_cache.dtype))
    return dims, max_q, total_q, H


def workspace_bytes_for(query, kv_cache, block_tables, seq_lens, max_seq_len, *, qo_indptr=None,
                        max_seq_len_q=None, return_lse=False):
    dims, max_q, _, _ = dims_for(query, kv_cache, block_tables, seq_lens, qo_indptr, max_seq_len_q)
    n = mla_decode_paged_workspace_size(dims, max_seq_len, max_q, return_lse)
    if n == 0:
        raise ValueError("shape rejected by the library (see mla_decode_paged status codes)")
    return n


def _device_scalar(name, v, device):
    if not isinstance(v, torch.Tensor):
        return None
    if v.dtype != torch.float32 or v.numel() != 1 or not v.is_cuda or v.device != device:
        raise TypeError(f"{name} as a tensor must be one float32 element on the query's device")
    return v


def decode(query, kv_cache, workspace_buffer, block_tables, seq_lens, max_seq_len, *, qo_indptr=None,
           max_seq_len_q=None, out=None, lse=None, return_lse=False, bmm1_scale=1.0, bmm2_scale=1.0,
           causal=True, sinks=None, dcp=None):
    """Batched paged MLA decode.  Returns out, or (out, lse) with return_lse.

    bmm1_scale / bmm2_scale: a float, or a one-element float32 device tensor
    read by the kernels at run time (so a captured graph follows updates).
    query may be float8_e4m3fn with a float8_e4m3fn cache (its q_scale folded
    into bmm1_scale by the caller): QK^T then runs on the fp8 matrix cores.
    sinks: None or a float32 device tensor [H] of per-head sink logits.
    dcp: None, or (seq_lens_global int32 device [B], cp_world, cp_rank) for the
    sequence-sharded partial mode (kv_cache / block_tables / seq_lens then hold
    this rank's rows; needs return_lse); merge the ranks with merge_partials.
    Sinks given with dcp enter rank 0's partial only."""
    for name, t in (("query", query), ("kv_cache", kv_cache), ("workspace_buffer", workspace_buffer),
                    ("block_tables", block_tables), ("seq_lens", seq_lens)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if query.dtype not in (torch.bfloat16, torch.float8_e4m3fn):
        raise TypeError("query must be bfloat16 (or float8_e4m3fn with a float8_e4m3fn cache)")
    q8 = query.dtype == torch.float8_e4m3fn
    if q8 and kv_cache.dtype != torch.float8_e4m3fn:
        raise TypeError("an fp8 query needs a float8_e4m3fn cache")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_tables and seq_lens must be int32")
    if qo_indptr is not None and (qo_indptr.dtype != torch.int32 or not qo_indptr.is_cuda):
        raise TypeError("qo_indptr must be an int32 device tensor")
    for name, t in (("kv_cache", kv_cache), ("workspace_buffer", workspace_buffer), ("block_tables", block_tables),
                    ("seq_lens", seq_lens), ("qo_indptr", qo_indptr)):
        if t is not None and t.device != query.device:
            raise ValueError(f"{name} must be on the query's device {query.device}")
    dims, max_q, total_q, H = dims_for(query, kv_cache, block_tables, seq_lens, qo_indptr, max_seq_len_q)
    out_shape = tuple(query.shape[:-1]) + (KV_LORA_RANK,)
    if out is None:
        out = torch.empty(out_shape, dtype=torch.bfloat16, device=query.device)
    elif tuple(out.shape) != out_shape or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous bfloat16 tensor of shape {out_shape}")
    if return_lse:
        lse_shape = tuple(query.shape[:-1])
        if lse is None:
            lse = torch.empty(lse_shape, dtype=torch.float32, device=query.device)
        elif tuple(lse.shape) != lse_shape or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError(f"lse must be a contiguous float32 tensor of shape {lse_shape}")
    else:
        lse = None
    ws_bytes = workspace_buffer.numel() * workspace_buffer.element_size()
    b1 = _device_scalar("bmm1_scale", bmm1_scale, query.device)
    b2 = _device_scalar("bmm2_scale", bmm2_scale, query.device)
    if sinks is not None and (sinks.dtype != torch.float32 or tuple(sinks.shape) != (H,) or not sinks.is_cuda
                              or not sinks.is_contiguous() or sinks.device != query.device):
        raise TypeError(f"sinks must be a contiguous float32 tensor of shape ({H},) on the query's device")
    if dcp is not None:
        lens_g, cp_world, cp_rank = dcp
        if (lens_g.dtype != torch.int32 or not lens_g.is_cuda or tuple(lens_g.shape) != tuple(seq_lens.shape)
                or not lens_g.is_contiguous() or lens_g.device != query.device):
            raise TypeError("dcp seq_lens_global must be a contiguous int32 tensor shaped like seq_lens on the "
                            "query's device")
        if not return_lse:
            raise ValueError("the sequence-sharded mode needs return_lse=True")
    if b1 is None and b2 is None and sinks is None and dcp is None and not q8:
        rc = mla_decode_paged(query, kv_cache, block_tables, seq_lens, qo_indptr, max_seq_len, max_q, bmm1_scale,
                              bmm2_scale, causal, out, lse, workspace_buffer, ws_bytes, dims)
    else:
        opts = MlaOptions(_ptr(b1), _ptr(b2), _ptr(sinks), None if dcp is None else _ptr(dcp[0]),
                          1 if dcp is None else int(dcp[1]), 0 if dcp is None else int(dcp[2]), 0, int(q8))
        rc = mla_decode_paged_ex(query, kv_cache, block_tables, seq_lens, qo_indptr, max_seq_len, max_q,
                                 1.0 if b1 is not None else bmm1_scale, 1.0 if b2 is not None else bmm2_scale,
                                 causal, out, lse, workspace_buffer, ws_bytes, dims, opts)
    if rc != MLA_OK:
        raise RuntimeError(f"mla_decode_paged failed: {mla_status_string(rc)} (status {rc})")
    return (out, lse) if return_lse else out


def _sparse_dims(query, kv_cache, indices):
    if kv_cache.dim() == 4:
        if kv_cache.shape[1] != 1:
            raise ValueError("rank-4 kv_cache must be [pages, 1, page_size, 576]")
        kv_cache = kv_cache.squeeze(1)
    if kv_cache.dim() != 3 or kv_cache.shape[-1] != D_QK:
        raise ValueError("kv_cache must be [pages, page_size, 576]")
    if query.dim() not in (3, 4) or query.shape[-1] != D_QK:
        raise ValueError("query must be [rows, H, 576] or [B, SQ, H, 576]")
    H = int(query.shape[-2])
    R = query.numel() // (H * D_QK)
    if indices.dim() != 2 or int(indices.shape[0]) != R:
        raise ValueError(f"indices must be [{R}, top_k] (one list per query row)")
    dims = make_dims(batch=R, num_heads=H, q_len_fixed=1, total_q=R, page_size=int(kv_cache.shape[1]),
                     num_pages=int(kv_cache.shape[0]), block_table_stride=int(indices.shape[1]),
                     kv_dtype=_kv_code(kv_cache.dtype))
    return dims, R, H


def sparse_workspace_bytes_for(query, kv_cache, indices, *, top_k=None, return_lse=False):
    dims, _, _ = _sparse_dims(query, kv_cache, indices)
    k = int(indices.shape[1]) if top_k is None else int(top_k)
    opts = MlaOptions(None, None, None, None, 1, 0, k)
    n = mla_decode_paged_ex_workspace_size(dims, 1, 1, return_lse, opts)
    if n == 0:
        raise ValueError("shape rejected by the library (see mla_decode_paged_ex status codes)")
    return n


def decode_sparse(query, kv_cache, workspace_buffer, indices, *, top_k=None, out=None, lse=None, return_lse=False,
                  bmm1_scale=1.0, bmm2_scale=1.0, sinks=None):
    """Sparse top-k MLA decode: every head of query row r attends to the cache
    rows listed in indices[r, :top_k] (int32 flat token ids page * page_size +
    slot; negative = empty).  The indices go to the C library as its
    block_tables with mla_decode_options_t.sparse_top_k = top_k (default: the
    row width).  Scales and sinks as in decode().  Returns out, or (out, lse)."""
    for name, t in (("query", query), ("kv_cache", kv_cache), ("workspace_buffer", workspace_buffer),
                    ("indices", indices)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if query.dtype != torch.bfloat16:
        raise TypeError("query must be bfloat16")
    if indices.dtype != torch.int32:
        raise TypeError("indices must be int32")
    dims, R, H = _sparse_dims(query, kv_cache, indices)
    k = int(indices.shape[1]) if top_k is None else int(top_k)
    out_shape = tuple(query.shape[:-1]) + (KV_LORA_RANK,)
    if out is None:
        out = torch.empty(out_shape, dtype=torch.bfloat16, device=query.device)
    elif tuple(out.shape) != out_shape or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous bfloat16 tensor of shape {out_shape}")
    if return_lse:
        lse_shape = tuple(query.shape[:-1])
        if lse is None:
            lse = torch.empty(lse_shape, dtype=torch.float32, device=query.device)
        elif tuple(lse.shape) != lse_shape or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError(f"lse must be a contiguous float32 tensor of shape {lse_shape}")
    else:
        lse = None
    b1 = _device_scalar("bmm1_scale", bmm1_scale, query.device)
    b2 = _device_scalar("bmm2_scale", bmm2_scale, query.device)
    if sinks is not None and (sinks.dtype != torch.float32 or tuple(sinks.shape) != (H,) or not sinks.is_cuda
                              or not sinks.is_contiguous() or sinks.device != query.device):
        raise TypeError(f"sinks must be a contiguous float32 tensor of shape ({H},) on the query's device")
    for name, t in (("kv_cache", kv_cache), ("workspace_buffer", workspace_buffer), ("indices", indices)):
        if t.device != query.device:
            raise ValueError(f"{name} must be on the query's device {query.device}")
    opts = MlaOptions(_ptr(b1), _ptr(b2), _ptr(sinks), None, 1, 0, k)
    ws_bytes = workspace_buffer.numel() * workspace_buffer.element_size()
    rc = mla_decode_paged_ex(query, kv_cache, indices, None, None, 1, 1, 1.0 if b1 is not None else bmm1_scale,
                             1.0 if b2 is not None else bmm2_scale, False, out, lse, workspace_buffer, ws_bytes,
                             dims, opts)
    if rc != MLA_OK:
        raise RuntimeError(f"mla_decode_paged_ex (sparse) failed: {mla_status_string(rc)} (status {rc})")
    return (out, lse) if return_lse else out


def merge_partials(outs, lses, out=None, lse=None):
    """Combine G partials of the same items: outs bf16 [G, ..., 512] and lses
    float32 [G, ...] (e.g. the ranks of a sequence-sharded decode, stacked).
    Returns (out bf16 [..., 512], lse float32 [...])."""
    if outs.dtype != torch.bfloat16 or lses.dtype != torch.float32 or not outs.is_cuda or not lses.is_cuda:
        raise TypeError("outs must be bf16 and lses float32 device tensors")
    if not outs.is_contiguous() or not lses.is_contiguous():
        raise ValueError("outs and lses must be contiguous")
    G = int(outs.shape[0])
    if tuple(outs.shape[:-1]) != tuple(lses.shape) or outs.shape[-1] != KV_LORA_RANK:
        raise ValueError("outs must be [G, ..., 512] and lses [G, ...] with matching leading shape")
    items = lses[0].numel()
    if out is None:
        out = torch.empty(tuple(outs.shape[1:]), dtype=torch.bfloat16, device=outs.device)
    if lse is None:
        lse = torch.empty(tuple(lses.shape[1:]), dtype=torch.float32, device=outs.device)
    rc = load_library().mla_merge_partials(outs.data_ptr(), lses.data_ptr(), G, items, out.data_ptr(),
                                           lse.data_ptr(), torch.cuda.current_stream().cuda_stream)
    if rc != MLA_OK:
        raise RuntimeError(f"mla_merge_partials failed: {mla_status_string(rc)} (status {rc})")
    return out, lse


# Bits of mla_decode_check_contract's result word (MLA_CONTRACT_* in include/mla_decode.h).
CONTRACT_BITS = {
    "seq_len": 1 << 0,
    "qo_start": 1 << 1,
    "qo_order": 1 << 2,
    "qo_end": 1 << 3,
    "q_len": 1 << 4,
    "causal": 1 << 5,
    "page_id": 1 << 6,
}


def check_contract(query, kv_cache, block_tables, seq_lens, max_seq_len, *, qo_indptr=None, max_seq_len_q=None,
                   causal=False):
    """Test and debugging aid: run the library's device-side check of the
    launch contract held in device memory (lengths, query offsets, causal
    lengths, page ids) for the arguments decode() would get, and return
    (set of violated rule names, lowest offending request or None).  Waits for
    the check to finish; it is not part of the decode path."""
    dims, max_q, _, _ = dims_for(query, kv_cache, block_tables, seq_lens, qo_indptr, max_seq_len_q)
    dev = seq_lens.device
    for name, t in (("block_tables", block_tables), ("seq_lens", seq_lens), ("qo_indptr", qo_indptr)):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous() or t.device != dev):
            raise TypeError(f"{name} must be a contiguous int32 tensor on {dev}")
    result = torch.zeros(2, dtype=torch.int32, device=dev)
    rc = load_library().mla_decode_check_contract(block_tables.data_ptr(), seq_lens.data_ptr(),
                                                  None if qo_indptr is None else qo_indptr.data_ptr(),
                                                  int(max_seq_len), int(max_q), int(bool(causal)), ctypes.byref(dims),
                                                  result.data_ptr(), torch.cuda.current_stream(dev).cuda_stream)
    if rc != MLA_OK:
        raise RuntimeError(f"mla_decode_check_contract failed: {mla_status_string(rc)} (status {rc})")
    bits, first = (int(v) & 0xFFFFFFFF for v in result.cpu().tolist())
    return {n for n, m in CONTRACT_BITS.items() if bits & m}, (first - 1 if first else None)


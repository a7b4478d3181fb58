"""Thin ctypes binding of libpagedattn.so (argument marshalling only).

Every function takes torch tensors that live on the GPU, checks their dtype,
shape and layout against each other, and passes their device pointers, the
sizes and torch's current HIP stream to the C ABI of ``include/pagedattn.h``.
All computation happens in the library's HIP kernels; there is no other path.
If the shared library has not been built, ``load_library`` raises.
"""

import ctypes
import math
import os

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so")

PA_F32, PA_F16, PA_BF16 = 0, 1, 2
_DTYPE_CODE = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}

KERNEL_AUTO, KERNEL_GENERIC, KERNEL_MFMA = 0, 1, 2

_lib = None

_VP = ctypes.c_void_p
_I = ctypes.c_int
_SIGNATURES = {
    "pa_version": (_I, []),
    "pa_status_string": (ctypes.c_char_p, [_I]),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_debug_select_kernel": (_I, [_I]),
    "pa_decode_kernel": (_I, [_I, _I, _I, _I]),
    "pa_decode_partition_size": (_I, [_I, _I, _I, _I, _I, _I, _I]),
    "pa_decode_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "pa_paged_attention_decode": (
        _I, [_VP, _VP, _VP, _VP, _VP, _VP,
             _I, _I, _I, _I, _I, _I, _I, _I, _I,
             ctypes.c_float, _I, _I, _VP, ctypes.c_size_t, _VP]),
    "pa_paged_attention_decode_noalloc": (
        _I, [_VP, _VP, _VP, _VP, _VP, _VP,
             _I, _I, _I, _I, _I, _I, _I, _I, _I,
             ctypes.c_float, _I, _I, _VP]),
    "pa_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "pa_decode_append": (
        _I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
             _I, _I, _I, _I, _I, _I, _I, _I, _I,
             ctypes.c_float, _I, _I, _VP, ctypes.c_size_t, _VP]),
    "pa_reshape_and_cache": (
        _I, [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _VP]),
    "pa_debug_gather_kv": (
        _I, [_VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _I, _I, _VP]),
    "pa_copy_blocks": (_I, [_VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _VP]),
    "pa_verify_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "pa_paged_attention_verify": (
        _I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP,
             _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I,
             ctypes.c_float, _I, _I, _VP, ctypes.c_size_t, _VP]),
    "pa_paged_attention_decode_fp8": (
        _I, [_VP, _VP, _VP, _VP, _VP, _VP,
             _I, _I, _I, _I, _I, _I, _I, _I, _I,
             ctypes.c_float, _I, ctypes.c_float, ctypes.c_float, _I, _VP, ctypes.c_size_t, _VP]),
    "pa_decode_append_fp8": (
        _I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
             _I, _I, _I, _I, _I, _I, _I, _I, _I,
             ctypes.c_float, _I, ctypes.c_float, ctypes.c_float, _I, _VP, ctypes.c_size_t, _VP]),
    "pa_reshape_and_cache_fp8": (
        _I, [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, ctypes.c_float, ctypes.c_float,
             _VP]),
    "pa_paged_attention_decode_i8": (
        _I, [_VP, _VP, _VP, _VP, _VP, _VP,
             _I, _I, _I, _I, _I, _I, _I, _I, _I,
             ctypes.c_float, _I, ctypes.c_float, ctypes.c_float, _I, _VP, ctypes.c_size_t, _VP]),
    "pa_decode_append_i8": (
        _I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
             _I, _I, _I, _I, _I, _I, _I, _I, _I,
             ctypes.c_float, _I, ctypes.c_float, ctypes.c_float, _I, _VP, ctypes.c_size_t, _VP]),
    "pa_reshape_and_cache_i8": (
        _I, [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, ctypes.c_float, ctypes.c_float,
             _VP]),
    "pa_pool_create": (_VP, [_I, _I]),
    "pa_pool_destroy": (None, [_VP]),
    "pa_pool_add_sequence": (_I, [_VP]),
    "pa_pool_fork": (_I, [_VP, _I]),
    "pa_pool_append": (_I, [_VP, _VP, _I, _VP, _VP, _VP]),
    "pa_pool_release": (_I, [_VP, _I]),
    "pa_pool_length": (_I, [_VP, _I]),
    "pa_pool_table": (_I, [_VP, _I, _VP, _I]),
    "pa_pool_refcount": (_I, [_VP, _I]),
    "pa_pool_free_blocks": (_I, [_VP]),
    "pa_check_slot_mapping": (_I, [_VP, _I, ctypes.c_int64]),
    "pa_bench_stream_read": (_I, [_VP, ctypes.c_size_t, _VP, _VP]),
    "pa_bench_copy": (_I, [_VP, _VP, ctypes.c_size_t, _VP]),
}


def load_library(path=None):
    """Load libpagedattn.so (once) and declare its C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(
            "libpagedattn.so not found at %s; build it with "
            "`python -m paged_kv_decode_attention_amd.build`" % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status, what):
    if status != 0:
        lib = load_library()
        raise RuntimeError("%s failed: %s (%s)" % (
            what, lib.pa_status_string(status).decode(), lib.pa_last_error().decode()))


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _gpu(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def dtype_code(dtype):
    if dtype not in _DTYPE_CODE:
        raise ValueError("unsupported dtype %s" % dtype)
    return _DTYPE_CODE[dtype]


def select_kernel(kind):
    """Pick the decode kernel family (KERNEL_AUTO / _GENERIC / _MFMA); returns
    the previous choice.  For comparing the two device paths in tests."""
    prev = load_library().pa_debug_select_kernel(int(kind))
    if prev < 0:
        _check(prev, "select_kernel")
    return prev


def decode_kernel(head_dim, block_size, gqa_group_size, dtype):
    """The kernel family a decode call of this shape runs now: KERNEL_GENERIC
    (vector ALU) or KERNEL_MFMA (matrix cores)."""
    k = load_library().pa_decode_kernel(int(head_dim), int(block_size), int(gqa_group_size),
                                        dtype_code(dtype))
    if k < 0:
        _check(k, "decode_kernel")
    return k


def decode_partition_size(num_seqs, num_kv_heads, gqa_group_size, head_dim, block_size,
                          max_context_len, dtype):
    return load_library().pa_decode_partition_size(
        num_seqs, num_kv_heads, gqa_group_size, head_dim, block_size, max_context_len,
        dtype_code(dtype))


def decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                          max_context_len, partition_size, dtype):
    n = load_library().pa_decode_workspace_size(
        num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len,
        partition_size, dtype_code(dtype))
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid sizes for the decode workspace")
    return n


FP8_CACHE_DTYPES = (torch.uint8, torch.float8_e4m3fn)
INT8_CACHE_DTYPES = (torch.int8,)
# 8-bit cache formats: accepted cache dtypes and their description
_CODES = {"fp8": (FP8_CACHE_DTYPES, "FP8 caches must be uint8 or float8_e4m3fn tensors of "
                                    "E4M3 codes"),
          "int8": (INT8_CACHE_DTYPES, "INT8 caches must be int8 tensors")}


def _decode_args(query, key_cache, value_cache, block_tables, context_lens, scale,
                 max_context_len, partition_size, out, workspace, kv8=None,
                 workspace_from_library=False):
    for t, n in ((query, "query"), (key_cache, "key_cache"), (value_cache, "value_cache"),
                 (block_tables, "block_tables"), (context_lens, "context_lens")):
        _gpu(t, n)
    if query.dim() != 3 or key_cache.dim() != 4 or key_cache.shape != value_cache.shape:
        raise ValueError("query must be [S,H,D] and caches [N,H_kv,BS,D] of one shape")
    S, H, D = query.shape
    N, H_kv, BS, D2 = key_cache.shape
    if D2 != D:
        raise ValueError("head_dim of query (%d) and caches (%d) differ" % (D, D2))
    if kv8 is not None:
        ok, msg = _CODES[kv8]
        if key_cache.dtype not in ok or value_cache.dtype not in ok:
            raise ValueError(msg)
    elif key_cache.dtype != query.dtype or value_cache.dtype != query.dtype:
        raise ValueError("query and caches must share one dtype")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [S, W] and context_lens [S]")
    if H_kv == 0 or H % H_kv:
        raise ValueError("num_heads %d is not a multiple of num_kv_heads %d" % (H, H_kv))
    W = block_tables.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if max_context_len is None:
        max_context_len = W * BS
    if out is None:
        out = torch.empty_like(query)
    else:
        _gpu(out, "out")
        if out.shape != query.shape or out.dtype != query.dtype:
            raise ValueError("out must match query in shape and dtype")
    ws_bytes = 0 if workspace_from_library else decode_workspace_size(
        S, H, H_kv, D, BS, max_context_len, partition_size, query.dtype)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=query.device)
    ws_ptr = _ptr(workspace) if workspace is not None else ctypes.c_void_p(0)
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    sizes = (S, H, H_kv, H // H_kv, D, BS, N, W, int(max_context_len))
    tail = (float(scale), dtype_code(query.dtype), int(partition_size), ws_ptr, ws_len,
            _stream(query.device))
    return out, sizes, tail


def _q8_tail(tail, k_scale, v_scale):
    # (scale, dtype, partition_size, ws, ws_len, stream) ->
    # (scale, dtype, k_scale, v_scale, partition_size, ws, ws_len, stream)
    return tail[:2] + (float(k_scale), float(v_scale)) + tail[2:]


def paged_attention_decode(query, key_cache, value_cache, block_tables, context_lens,
                           scale=None, *, max_context_len=None, partition_size=0,
                           out=None, workspace=None):
    """Single-step decode attention over a paged KV cache.

    query [S, H, D]; key_cache/value_cache [N, H_kv, BS, D] (same dtype);
    block_tables [S, W] int32; context_lens [S] int32.  The GQA group size is
    H / H_kv.  max_context_len defaults to W * BS (no device sync).  Returns
    out [S, H, D] in the query dtype.
    """
    out, sizes, tail = _decode_args(query, key_cache, value_cache, block_tables, context_lens,
                                    scale, max_context_len, partition_size, out, workspace)
    status = load_library().pa_paged_attention_decode(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), *sizes, *tail)
    _check(status, "paged_attention_decode")
    return out


def paged_attention_decode_noalloc(query, key_cache, value_cache, block_tables, context_lens,
                                   scale=None, *, max_context_len=None, partition_size=0,
                                   out=None):
    """paged_attention_decode with the library's own per-GPU device array as
    the workspace (pa_paged_attention_decode_noalloc): no allocation by the
    library; `out` given, nothing is allocated at all.  Calls that overlap in
    time on one GPU must not be made (they share the array)."""
    out, sizes, tail = _decode_args(query, key_cache, value_cache, block_tables, context_lens,
                                    scale, max_context_len, partition_size, out, None,
                                    workspace_from_library=True)
    scale_, dt, P, _, _, stream = tail
    _check(load_library().pa_paged_attention_decode_noalloc(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), *sizes, scale_, dt, P, stream), "paged_attention_decode_noalloc")
    return out


def decode_append(query, key, value, key_cache, value_cache, block_tables, context_lens,
                  scale=None, *, max_context_len=None, partition_size=0, out=None,
                  workspace=None):
    """One decode step: store each sequence's newest token key/value [S, H_kv, D]
    at its history position context_lens[b] - 1 (slot from the block table),
    then attend.  context_lens count the new token.  In place on the caches."""
    out, sizes, tail = _decode_args(query, key_cache, value_cache, block_tables, context_lens,
                                    scale, max_context_len, partition_size, out, workspace)
    for t, n in ((key, "key"), (value, "value")):
        _gpu(t, n)
    S, H_kv, D = query.shape[0], key_cache.shape[1], query.shape[2]
    if key.shape != (S, H_kv, D) or value.shape != key.shape:
        raise ValueError("key and value must be [S, H_kv, D]")
    if key.dtype != query.dtype or value.dtype != query.dtype:
        raise ValueError("key/value must share the query dtype")
    status = load_library().pa_decode_append(
        _ptr(out), _ptr(query), _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
        _ptr(block_tables), _ptr(context_lens), *sizes, *tail)
    _check(status, "decode_append")
    return out


def check_slot_mapping(slot_mapping, num_slots):
    """Raise RuntimeError unless every non-negative slot of slot_mapping (a
    tensor on any device, or an array; int64 [T]) is below num_slots and no
    two tokens share one.  Copies the mapping to the host (synchronising)."""
    if isinstance(slot_mapping, torch.Tensor):
        slot_mapping = slot_mapping.detach().cpu().numpy()
    host = np.ascontiguousarray(slot_mapping, dtype=np.int64).reshape(-1)
    _check(load_library().pa_check_slot_mapping(host.ctypes.data_as(ctypes.c_void_p), host.size,
                                                int(num_slots)), "check_slot_mapping")


def _checking_slots(check_slots):
    """check_slots if given, else whether PAGEDATTN_CHECK_SLOTS=1 is set."""
    if check_slots is None:
        return os.environ.get("PAGEDATTN_CHECK_SLOTS") == "1"
    return bool(check_slots)


def reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, *, check_slots=None):
    """Store key/value [T, H_kv, D] into the caches at slot_mapping [T] (int64;
    negative = skip).  In place on the caches.  With check_slots (default:
    the PAGEDATTN_CHECK_SLOTS=1 environment setting), the mapping is first
    checked on the host by check_slot_mapping."""
    for t, n in ((key, "key"), (value, "value"), (key_cache, "key_cache"),
                 (value_cache, "value_cache"), (slot_mapping, "slot_mapping")):
        _gpu(t, n)
    if key.shape != value.shape or key.dim() != 3:
        raise ValueError("key and value must be [T, H_kv, D] of one shape")
    if key_cache.shape != value_cache.shape or key_cache.dim() != 4:
        raise ValueError("caches must be [N, H_kv, BS, D] of one shape")
    T, H_kv, D = key.shape
    N, H_kv2, BS, D2 = key_cache.shape
    if (H_kv, D) != (H_kv2, D2):
        raise ValueError("new tokens and caches disagree in KV heads or head_dim")
    if len({key.dtype, value.dtype, key_cache.dtype, value_cache.dtype}) != 1:
        raise ValueError("key, value and caches must share one dtype")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be int64 [T]")
    if _checking_slots(check_slots):
        check_slot_mapping(slot_mapping, N * BS)
    status = load_library().pa_reshape_and_cache(
        _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache), _ptr(slot_mapping),
        T, H_kv, D, BS, N, dtype_code(key.dtype), _stream(key.device))
    _check(status, "reshape_and_cache")


def debug_gather_kv(key_cache, value_cache, block_tables, context_lens, seq,
                    max_context_len=None, k_out=None, v_out=None):
    """Contiguous [H_kv, max_context_len, D] copies of sequence `seq`'s history
    (rows >= its length are left as given), via the kernels' address code."""
    for t, n in ((key_cache, "key_cache"), (value_cache, "value_cache"),
                 (block_tables, "block_tables"), (context_lens, "context_lens")):
        _gpu(t, n)
    N, H_kv, BS, D = key_cache.shape
    S, W = block_tables.shape
    if max_context_len is None:
        max_context_len = W * BS
    if k_out is None:
        k_out = torch.zeros((H_kv, max_context_len, D), dtype=key_cache.dtype,
                            device=key_cache.device)
    if v_out is None:
        v_out = torch.zeros_like(k_out)
    status = load_library().pa_debug_gather_kv(
        _ptr(k_out), _ptr(v_out), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), int(seq), S, H_kv, D, BS, N, W, int(max_context_len),
        dtype_code(key_cache.dtype), _stream(key_cache.device))
    _check(status, "debug_gather_kv")
    return k_out, v_out


def stream_read(src, sink):
    """Read all of `src` (a GPU tensor, bytes multiple of 16) once."""
    _check(load_library().pa_bench_stream_read(
        _ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(src.device)),
        "stream_read")


def copy_bytes(dst, src):
    """Copy src to dst (same byte size, multiple of 16) with a plain kernel."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst too small")
    _check(load_library().pa_bench_copy(_ptr(dst), _ptr(src), n, _stream(src.device)),
           "copy_bytes")


def paged_attention_verify(query, key_cache, value_cache, block_tables, context_lens,
                           query_start, max_query_len, scale=None, *, max_context_len=None,
                           partition_size=0, out=None, workspace=None):
    """Decode with several new query tokens per sequence (speculative verify).

    query [total_q, H, D]: sequence b owns rows query_start[b] ..
    query_start[b+1] - 1 (query_start [S+1] int32 on the GPU), its q_b newest
    tokens, already in the caches; row i attends history positions
    t <= context_lens[b] - q_b + i.  max_query_len bounds every q_b.
    """
    for t, n in ((query, "query"), (key_cache, "key_cache"), (value_cache, "value_cache"),
                 (block_tables, "block_tables"), (context_lens, "context_lens"),
                 (query_start, "query_start")):
        _gpu(t, n)
    if query.dim() != 3 or key_cache.dim() != 4 or key_cache.shape != value_cache.shape:
        raise ValueError("query must be [total_q,H,D] and caches [N,H_kv,BS,D] of one shape")
    if key_cache.dtype != query.dtype or value_cache.dtype != query.dtype:
        raise ValueError("query and caches must share one dtype")
    for t, n in ((block_tables, "block_tables"), (context_lens, "context_lens"),
                 (query_start, "query_start")):
        if t.dtype != torch.int32:
            raise ValueError("%s must be int32" % n)
    TQ, H, D = query.shape
    N, H_kv, BS, D2 = key_cache.shape
    S = context_lens.shape[0]
    if D2 != D or block_tables.dim() != 2 or block_tables.shape[0] != S or \
            query_start.shape != (S + 1,):
        raise ValueError("shapes disagree: block_tables [S, W], query_start [S+1]")
    if H_kv == 0 or H % H_kv:
        raise ValueError("num_heads %d is not a multiple of num_kv_heads %d" % (H, H_kv))
    W = block_tables.shape[1]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    max_context_len = W * BS if max_context_len is None else max_context_len
    if out is None:
        out = torch.empty_like(query)
    lib = load_library()
    need = lib.pa_verify_workspace_size(TQ, H, H_kv, D, BS, int(max_context_len),
                                        int(partition_size), dtype_code(query.dtype))
    if need == ctypes.c_size_t(-1).value:
        raise ValueError("invalid sizes for the verify workspace")
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=query.device)
    _check(lib.pa_paged_attention_verify(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), _ptr(query_start), S, TQ, int(max_query_len), H, H_kv, H // H_kv, D,
        BS, N, W, int(max_context_len), float(scale), dtype_code(query.dtype),
        int(partition_size), _ptr(workspace), workspace.numel(), _stream(query.device)),
        "paged_attention_verify")
    return out


def _decode_q8(kv8, query, key_cache, value_cache, block_tables, context_lens, k_scale,
               v_scale, scale, max_context_len, partition_size, out, workspace):
    out, sizes, tail = _decode_args(query, key_cache, value_cache, block_tables, context_lens,
                                    scale, max_context_len, partition_size, out, workspace,
                                    kv8=kv8)
    name = "paged_attention_decode_" + ("fp8" if kv8 == "fp8" else "i8")
    status = getattr(load_library(), "pa_" + name)(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), *sizes, *_q8_tail(tail, k_scale, v_scale))
    _check(status, name)
    return out


def _decode_append_q8(kv8, query, key, value, key_cache, value_cache, block_tables,
                      context_lens, k_scale, v_scale, scale, max_context_len, partition_size,
                      out, workspace):
    out, sizes, tail = _decode_args(query, key_cache, value_cache, block_tables, context_lens,
                                    scale, max_context_len, partition_size, out, workspace,
                                    kv8=kv8)
    for t, n in ((key, "key"), (value, "value")):
        _gpu(t, n)
    S, H_kv, D = query.shape[0], key_cache.shape[1], query.shape[2]
    if key.shape != (S, H_kv, D) or value.shape != key.shape:
        raise ValueError("key and value must be [S, H_kv, D]")
    if key.dtype != query.dtype or value.dtype != query.dtype:
        raise ValueError("key/value must share the query dtype")
    name = "decode_append_" + ("fp8" if kv8 == "fp8" else "i8")
    status = getattr(load_library(), "pa_" + name)(
        _ptr(out), _ptr(query), _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
        _ptr(block_tables), _ptr(context_lens), *sizes, *_q8_tail(tail, k_scale, v_scale))
    _check(status, name)
    return out


def _reshape_and_cache_q8(kv8, key, value, key_cache, value_cache, slot_mapping, k_scale,
                          v_scale, check_slots):
    for t, n in ((key, "key"), (value, "value"), (key_cache, "key_cache"),
                 (value_cache, "value_cache"), (slot_mapping, "slot_mapping")):
        _gpu(t, n)
    if key.shape != value.shape or key.dim() != 3 or key.dtype != value.dtype:
        raise ValueError("key and value must be [T, H_kv, D] of one shape and dtype")
    if key_cache.shape != value_cache.shape or key_cache.dim() != 4:
        raise ValueError("caches must be [N, H_kv, BS, D] of one shape")
    ok, msg = _CODES[kv8]
    if key_cache.dtype not in ok or value_cache.dtype not in ok:
        raise ValueError(msg)
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (key.shape[0],):
        raise ValueError("slot_mapping must be [T] int64")
    T, H_kv, D = key.shape
    N, H_kv2, BS, D2 = key_cache.shape
    if (H_kv, D) != (H_kv2, D2):
        raise ValueError("new tokens and caches disagree in KV heads or head_dim")
    if _checking_slots(check_slots):
        check_slot_mapping(slot_mapping, N * BS)
    name = "reshape_and_cache_" + ("fp8" if kv8 == "fp8" else "i8")
    _check(getattr(load_library(), "pa_" + name)(
        _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache), _ptr(slot_mapping), T, H_kv,
        D, BS, N, dtype_code(key.dtype), float(k_scale), float(v_scale),
        _stream(key.device)), name)


def paged_attention_decode_fp8(query, key_cache, value_cache, block_tables, context_lens,
                               k_scale, v_scale, scale=None, *, max_context_len=None,
                               partition_size=0, out=None, workspace=None):
    """paged_attention_decode over caches of OCP FP8 E4M3 codes (uint8 or
    float8_e4m3fn [N, H_kv, BS, D]); a code stands for decode(code) * k_scale
    (keys) or * v_scale (values).  query/out bf16 or f16; the shapes of the
    matrix-core kernel (head_dim 64/128/256, block size 8-64, GQA group up to
    16, or 32 at head_dim 64/128)."""
    return _decode_q8("fp8", query, key_cache, value_cache, block_tables, context_lens,
                      k_scale, v_scale, scale, max_context_len, partition_size, out, workspace)


def decode_append_fp8(query, key, value, key_cache, value_cache, block_tables, context_lens,
                      k_scale, v_scale, scale=None, *, max_context_len=None, partition_size=0,
                      out=None, workspace=None):
    """decode_append on E4M3 caches: the newest token's key/value (query
    dtype) are quantised with k_scale / v_scale as they are stored."""
    return _decode_append_q8("fp8", query, key, value, key_cache, value_cache, block_tables,
                             context_lens, k_scale, v_scale, scale, max_context_len,
                             partition_size, out, workspace)


def reshape_and_cache_fp8(key, value, key_cache, value_cache, slot_mapping, k_scale, v_scale, *,
                          check_slots=None):
    """Quantise key/value [T, H_kv, D] (f32, f16 or bf16) to E4M3 with the
    given scales and store them at slot_mapping [T] in the uint8 /
    float8_e4m3fn caches [N, H_kv, BS, D].  check_slots as for
    reshape_and_cache."""
    _reshape_and_cache_q8("fp8", key, value, key_cache, value_cache, slot_mapping, k_scale,
                          v_scale, check_slots)


def paged_attention_decode_i8(query, key_cache, value_cache, block_tables, context_lens,
                              k_scale, v_scale, scale=None, *, max_context_len=None,
                              partition_size=0, out=None, workspace=None):
    """paged_attention_decode over caches of signed INT8 codes (int8 [N, H_kv,
    BS, D]); code c stands for c * k_scale (keys) or c * v_scale (values).
    Query dtypes and shapes as for paged_attention_decode_fp8."""
    return _decode_q8("int8", query, key_cache, value_cache, block_tables, context_lens,
                      k_scale, v_scale, scale, max_context_len, partition_size, out, workspace)


def decode_append_i8(query, key, value, key_cache, value_cache, block_tables, context_lens,
                     k_scale, v_scale, scale=None, *, max_context_len=None, partition_size=0,
                     out=None, workspace=None):
    """decode_append on INT8 caches: the newest token's key/value (query
    dtype) are quantised with k_scale / v_scale as they are stored."""
    return _decode_append_q8("int8", query, key, value, key_cache, value_cache, block_tables,
                             context_lens, k_scale, v_scale, scale, max_context_len,
                             partition_size, out, workspace)


def reshape_and_cache_i8(key, value, key_cache, value_cache, slot_mapping, k_scale, v_scale, *,
                         check_slots=None):
    """Quantise key/value [T, H_kv, D] (f32, f16 or bf16) to INT8 codes
    (nearest integer of x / scale, ties to even, clamped to +-127, NaN to 0)
    and store them at slot_mapping [T] in the int8 caches [N, H_kv, BS, D].
    check_slots as for reshape_and_cache."""
    _reshape_and_cache_q8("int8", key, value, key_cache, value_cache, slot_mapping, k_scale,
                          v_scale, check_slots)


def copy_blocks(key_cache, value_cache, block_pairs):
    """key_cache[dst] = key_cache[src] and the same for value_cache, for each
    row (src, dst) of block_pairs ([n, 2] int32 on the GPU): the copy behind
    copy-on-write (see BlockPool.append)."""
    _gpu(key_cache, "key_cache")
    _gpu(value_cache, "value_cache")
    _gpu(block_pairs, "block_pairs")
    if key_cache.shape != value_cache.shape or key_cache.dtype != value_cache.dtype:
        raise ValueError("key_cache and value_cache must match")
    if block_pairs.dtype != torch.int32 or block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [n, 2] int32")
    N, H_kv, BS, D = key_cache.shape
    _check(load_library().pa_copy_blocks(
        _ptr(key_cache), _ptr(value_cache), _ptr(block_pairs), block_pairs.shape[0], H_kv, D,
        BS, N, dtype_code(key_cache.dtype), _stream(key_cache.device)), "copy_blocks")


class BlockPool:
    """The library's host-side block pool (pa_pool_* of pagedattn.h): block
    tables with reference counts and copy-on-write of shared partial blocks.
    Arrays cross the boundary as NumPy host arrays."""

    def __init__(self, num_blocks, block_size):
        self._np = np
        lib = load_library()
        self._lib = lib
        self._h = lib.pa_pool_create(int(num_blocks), int(block_size))
        if not self._h:
            raise RuntimeError("pa_pool_create failed: " + lib.pa_last_error().decode())
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self):
        if self._h:
            self._lib.pa_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _ok(self, r, what):
        if r < 0:
            _check(r, what)
        return r

    def add_sequence(self):
        return self._ok(self._lib.pa_pool_add_sequence(self._h), "pool add_sequence")

    def fork(self, seq):
        return self._ok(self._lib.pa_pool_fork(self._h, int(seq)), "pool fork")

    def append(self, seqs):
        """One new token for each sequence id in seqs, in order.  Returns
        (slots int64 [n], copy pairs int32 [c, 2]); run copy_blocks on the
        pairs before storing the tokens at the slots."""
        np = self._np
        ids = np.ascontiguousarray(seqs, dtype=np.int32)
        n = len(ids)
        slots = np.zeros(n, dtype=np.int64)
        pairs = np.zeros((max(n, 1), 2), dtype=np.int32)
        count = ctypes.c_int(0)
        _check(self._lib.pa_pool_append(
            self._h, ids.ctypes.data_as(_VP), n, slots.ctypes.data_as(_VP),
            pairs.ctypes.data_as(_VP), ctypes.byref(count)), "pool append")
        return slots, pairs[:count.value].copy()

    def release(self, seq):
        _check(self._lib.pa_pool_release(self._h, int(seq)), "pool release")

    def length(self, seq):
        return self._ok(self._lib.pa_pool_length(self._h, int(seq)), "pool length")

    def table(self, seq):
        np = self._np
        n = self._ok(self._lib.pa_pool_table(self._h, int(seq), None, 0), "pool table")
        out = np.zeros(max(n, 1), dtype=np.int32)
        self._lib.pa_pool_table(self._h, int(seq), out.ctypes.data_as(_VP), n)
        return out[:n].copy()

    def refcount(self, block):
        return self._ok(self._lib.pa_pool_refcount(self._h, int(block)), "pool refcount")

    def free_blocks(self):
        return self._ok(self._lib.pa_pool_free_blocks(self._h), "pool free_blocks")

"""ctypes binding of libpa.so (include/pa.h): argument marshalling only.

Every function here takes torch tensors, checks device / dtype / contiguity,
passes ``data_ptr()`` values and torch's current HIP stream to the C entry
point of the same name, and raises ``PaError`` on a non-OK status. All work
runs in the HIP kernels behind the C ABI; there is no fallback path. If the
library has not been built, the first call raises.
"""

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpa.so")

PA_DTYPE_F32 = 0
PA_DTYPE_BF16 = 1

PA_DTYPE_FP8_E4M3 = 2

STATUS_NAMES = {
    0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_SHAPE", 3: "PA_ERR_UNSUPPORTED",
    4: "PA_ERR_ALIGN", 5: "PA_ERR_WORKSPACE", 6: "PA_ERR_HIP", 7: "PA_ERR_OUT_OF_BLOCKS",
    8: "PA_ERR_STATE", 9: "PA_ERR_NOMEM",
}

# Exported symbols and their C signatures (mirrors include/pa.h).
_i32, _i64, _sz, _vp, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
SIGNATURES = {
    "pa_reshape_and_cache": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64, _i32, _vp]),
    "pa_decode_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode_workspace_init": (_i32, [_vp, _sz, _vp]),
    "pa_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i64,
                         _i32, _f32, _i32, _vp, _sz, _vp]),
    "pa_decode_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                 _i32, _i64, _i32, _f32, _i32, _vp]),
    "pa_decode_noalloc_max_bytes": (_sz, []),
    "pa_decode_shared_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                              _i32]),
    "pa_decode_shared": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                _i32, _i32, _i32, _i32, _i32, _i32, _i64, _i32, _f32, _i32, _vp,
                                _sz, _vp]),
    "pa_find_shared_prefixes": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "pa_reshape_and_cache_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                        _i64, _i32, _vp]),
    "pa_decode_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                             _i32, _i64, _i32, _f32, _i32, _vp, _sz, _vp]),
    "pa_prefill_chunk_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_prefill_chunk": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                _i32, _i32, _i32, _i64, _i32, _f32, _i32, _vp, _sz, _vp]),
    "pa_prefill_chunk_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                    _i32, _i32, _i32, _i32, _i32, _i32, _i64, _i32, _f32, _i32,
                                    _vp, _sz, _vp]),
    "pa_copy_blocks": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64, _i32, _vp]),
    "pa_bm_create": (_i32, [_i64, _i32, _i32, ctypes.POINTER(_vp)]),
    "pa_bm_destroy": (None, [_vp]),
    "pa_bm_add": (_i32, [_vp, _i64]),
    "pa_bm_fork": (_i32, [_vp, _i64, _i64]),
    "pa_bm_append": (_i32, [_vp, _i64, _i32, _vp]),
    "pa_bm_free": (_i32, [_vp, _i64]),
    "pa_bm_num_free": (_i64, [_vp]),
    "pa_bm_length": (_i64, [_vp, _i64]),
    "pa_bm_blocks_needed": (_i64, [_vp, _i64, _i32]),
    "pa_bm_refcount": (_i32, [_vp, _i64]),
    "pa_bm_table": (_i32, [_vp, _i64, _vp, _i32]),
    "pa_bm_tables": (_i32, [_vp, _vp, _i32, _vp, _i32, _vp]),
    "pa_bm_take_copies": (_i64, [_vp, _vp, _i64]),
    "pa_swap_out": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64, _i64, _i32,
                           _vp]),
    "pa_swap_in": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64, _i64, _i32,
                          _vp]),
    "pa_engine_create": (_i32, [_vp, _vp, _vp, _vp, _i32, _vp, ctypes.POINTER(_vp)]),
    "pa_engine_destroy": (None, [_vp]),
    "pa_engine_done": (_i32, [_vp]),
    "pa_engine_plan": (_i32, [_vp, _vp]),
    "pa_engine_execute": (_i32, [_vp]),
    "pa_engine_iterations": (_i64, [_vp]),
    "pa_engine_graph_launches": (_i64, [_vp]),
    "pa_sched_create": (_i32, [_vp, _vp, _vp, _i32, ctypes.POINTER(_vp)]),
    "pa_sched_destroy": (None, [_vp]),
    "pa_sched_done": (_i32, [_vp]),
    "pa_sched_step": (_i32, [_vp, _vp]),
    "pa_sched_blocks": (_vp, [_vp]),
    "pa_status_string": (ctypes.c_char_p, [_i32]),
    "pa_version": (_i32, []),
}


class PaError(RuntimeError):
    def __init__(self, fn, status, message):
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)} ({message})")
        self.status = status


_lib = None
_lock = threading.Lock()


def lib():
    """The loaded libpa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is missing: build it with "
                        "`python -m paged_kv_cache_215_amd.build` (no fallback exists)")
                handle = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in SIGNATURES.items():
                    fn = getattr(handle, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = handle
    return _lib


def _check(fn, status):
    if status != 0:
        msg = lib().pa_status_string(status).decode()
        raise PaError(fn, status, msg)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return PA_DTYPE_BF16
    if t.dtype == torch.float32:
        return PA_DTYPE_F32
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PA_DTYPE_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(*tensors):
    dev = tensors[0].device
    for t in tensors:
        if t.device.type != "cuda":
            raise ValueError("tensors must live on the GPU")
        if t.device != dev:
            raise ValueError("tensors must be on one device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return dev


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def pa_reshape_and_cache(key, value, key_cache, value_cache, slot_mapping):
    """Write token t's K/V rows into slot slot_mapping[t] of the caches (in place)."""
    dev = _dev(key, value, key_cache, value_cache, slot_mapping)
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    if key.dtype != key_cache.dtype or value.dtype != value_cache.dtype or key.dtype != value.dtype:
        raise TypeError("key/value and cache dtypes must match")
    num_tokens, num_kv_heads, head_dim = key.shape
    num_blocks, _, block_size, _ = key_cache.shape
    _check("pa_reshape_and_cache", lib().pa_reshape_and_cache(
        _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache), _ptr(slot_mapping),
        num_tokens, num_kv_heads, head_dim, block_size, num_blocks, _dtype_code(key_cache),
        _stream(dev)))


def pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                             max_context_len):
    return int(lib().pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                              block_size, max_context_len))


def pa_decode_workspace_init(workspace):
    """Zero-fill a decode workspace on the current stream (needed once)."""
    dev = _dev(workspace)
    _check("pa_decode_workspace_init", lib().pa_decode_workspace_init(
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev)))


def decode_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     max_context_len, device):
    """A zero-filled decode workspace for these sizes, reusable across calls."""
    need = pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                    max_context_len)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    pa_decode_workspace_init(ws)
    return ws


def pa_decode(query, key_cache, value_cache, block_tables, context_lens, scale,
              max_context_len, out=None, workspace=None):
    """Decode attention over the paged cache; returns float32 [S, Hq, d]."""
    dev = _dev(query, key_cache, value_cache, block_tables, context_lens)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    num_seqs, num_q_heads, head_dim = query.shape
    num_blocks, num_kv_heads, block_size, _ = key_cache.shape
    if out is None:
        out = torch.empty((num_seqs, num_q_heads, head_dim), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = decode_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                     max_context_len, dev)
    _dev(out, workspace)
    _check("pa_decode", lib().pa_decode(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
        block_tables.shape[1], num_blocks, int(max_context_len), float(scale),
        _dtype_code(query), _ptr(workspace), workspace.numel(), _stream(dev)))
    return out


def pa_decode_noalloc(query, key_cache, value_cache, block_tables, context_lens, scale,
                      max_context_len, out):
    """pa_decode on the library's static scratch: no workspace, nothing
    allocated (``out``, float32 [S, Hq, d], is the caller's)."""
    dev = _dev(query, key_cache, value_cache, block_tables, context_lens, out)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    num_seqs, num_q_heads, head_dim = query.shape
    num_blocks, num_kv_heads, block_size, _ = key_cache.shape
    _check("pa_decode_noalloc", lib().pa_decode_noalloc(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
        block_tables.shape[1], num_blocks, int(max_context_len), float(scale),
        _dtype_code(query), _stream(dev)))
    return out


def find_shared_prefixes(block_tables, context_lens, block_size, min_blocks=1):
    """Copy-on-write groups of a decode batch from its host block tables and
    lengths (numpy int32 arrays): (cu_groups, prefix_lens, max_group_size,
    max_prefix_len) as numpy int32 arrays and ints; no groups -> empty arrays."""
    import numpy as np
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    S = int(ctx.size)
    cu = np.zeros(S + 1, dtype=np.int32)
    pl = np.zeros(max(S, 1), dtype=np.int32)
    mg, mp = ctypes.c_int32(0), ctypes.c_int32(0)
    g = lib().pa_find_shared_prefixes(bt.ctypes.data_as(_vp), ctx.ctypes.data_as(_vp), S,
                                      bt.shape[1], block_size, min_blocks,
                                      cu.ctypes.data_as(_vp), pl.ctypes.data_as(_vp),
                                      ctypes.byref(mg), ctypes.byref(mp))
    if g < 0:
        raise ValueError("pa_find_shared_prefixes: invalid arguments")
    if g == 0:
        return cu[:0], pl[:0], 0, 0
    return cu[:g + 1].copy(), pl[:g].copy(), int(mg.value), int(mp.value)


def pa_decode_shared_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                    max_context_len, num_groups, max_group_size, max_prefix_len):
    return int(lib().pa_decode_shared_workspace_size(num_seqs, num_q_heads, num_kv_heads,
                                                     head_dim, block_size, max_context_len,
                                                     num_groups, max_group_size, max_prefix_len))


def decode_shared_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                            max_context_len, num_groups, max_group_size, max_prefix_len, device):
    """An initialised workspace for pa_decode_shared, reusable across calls."""
    need = pa_decode_shared_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                           block_size, max_context_len, num_groups,
                                           max_group_size, max_prefix_len)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    pa_decode_workspace_init(ws)
    return ws


def pa_decode_shared(query, key_cache, value_cache, block_tables, context_lens, cu_groups,
                     prefix_lens, max_group_size, max_prefix_len, scale, max_context_len,
                     k_scale=None, v_scale=None, out=None, workspace=None):
    """Decode over a batch with copy-on-write groups (cu_groups, prefix_lens:
    int32 device tensors); an FP8 cache (uint8 codes) takes k_scale / v_scale.
    Returns float32 [S, Hq, d]."""
    fp8 = key_cache.dtype in (torch.uint8, torch.float8_e4m3fn)
    tensors = [query, key_cache, value_cache, block_tables, context_lens, cu_groups, prefix_lens]
    if fp8:
        _scales(k_scale, v_scale)
        tensors += [k_scale, v_scale]
    dev = _dev(*tensors)
    for t in (block_tables, context_lens, cu_groups, prefix_lens):
        if t.dtype != torch.int32:
            raise TypeError("tables, lengths and group arrays must be int32")
    num_seqs, num_q_heads, head_dim = query.shape
    num_blocks, num_kv_heads, block_size, _ = key_cache.shape
    num_groups = prefix_lens.numel()
    if out is None:
        out = torch.empty((num_seqs, num_q_heads, head_dim), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = decode_shared_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                            block_size, max_context_len, num_groups,
                                            max_group_size, max_prefix_len, dev)
    _dev(out, workspace)
    _check("pa_decode_shared", lib().pa_decode_shared(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
        _ptr(k_scale if fp8 else None), _ptr(v_scale if fp8 else None), _ptr(block_tables),
        _ptr(context_lens), _ptr(cu_groups), _ptr(prefix_lens), num_groups, int(max_group_size),
        int(max_prefix_len), num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
        block_tables.shape[1], num_blocks, int(max_context_len), float(scale),
        PA_DTYPE_FP8_E4M3 if fp8 else _dtype_code(key_cache), _ptr(workspace), workspace.numel(),
        _stream(dev)))
    return out


def _fp8_cache(t):
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError("an FP8 cache holds E4M3 codes (uint8 or float8_e4m3fn)")


def _scales(*ts):
    for t in ts:
        if t.dtype != torch.float32:
            raise TypeError("FP8 scales are float32 [num_kv_heads]")


def pa_reshape_and_cache_fp8(key, value, key_cache, value_cache, slot_mapping, k_scale, v_scale):
    """Quantize token t's K/V rows to E4M3 with per-head scales and write them
    into slot slot_mapping[t] of the FP8 caches (in place)."""
    dev = _dev(key, value, key_cache, value_cache, slot_mapping, k_scale, v_scale)
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    _fp8_cache(key_cache)
    _fp8_cache(value_cache)
    _scales(k_scale, v_scale)
    if key.dtype != value.dtype:
        raise TypeError("key and value dtypes must match")
    num_tokens, num_kv_heads, head_dim = key.shape
    num_blocks, _, block_size, _ = key_cache.shape
    if k_scale.numel() != num_kv_heads or v_scale.numel() != num_kv_heads:
        raise ValueError("one scale per KV head")
    _check("pa_reshape_and_cache_fp8", lib().pa_reshape_and_cache_fp8(
        _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache), _ptr(slot_mapping),
        _ptr(k_scale), _ptr(v_scale), num_tokens, num_kv_heads, head_dim, block_size,
        num_blocks, _dtype_code(key), _stream(dev)))


def pa_decode_fp8(query, key_cache, value_cache, k_scale, v_scale, block_tables, context_lens,
                  scale, max_context_len, out=None, workspace=None):
    """Decode attention over an FP8 (E4M3) paged cache; returns float32 [S, Hq, d]."""
    dev = _dev(query, key_cache, value_cache, k_scale, v_scale, block_tables, context_lens)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    _fp8_cache(key_cache)
    _fp8_cache(value_cache)
    _scales(k_scale, v_scale)
    num_seqs, num_q_heads, head_dim = query.shape
    num_blocks, num_kv_heads, block_size, _ = key_cache.shape
    if k_scale.numel() != num_kv_heads or v_scale.numel() != num_kv_heads:
        raise ValueError("one scale per KV head")
    if out is None:
        out = torch.empty((num_seqs, num_q_heads, head_dim), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = decode_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                     max_context_len, dev)
    _dev(out, workspace)
    _check("pa_decode_fp8", lib().pa_decode_fp8(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_tables), _ptr(context_lens), num_seqs, num_q_heads, num_kv_heads, head_dim,
        block_size, block_tables.shape[1], num_blocks, int(max_context_len), float(scale),
        _dtype_code(query), _ptr(workspace), workspace.numel(), _stream(dev)))
    return out


def pa_prefill_chunk_workspace_size(num_seqs, total_q, max_q_len, num_q_heads, num_kv_heads,
                                    head_dim, block_size, max_context_len):
    return int(lib().pa_prefill_chunk_workspace_size(num_seqs, total_q, max_q_len, num_q_heads,
                                                     num_kv_heads, head_dim, block_size,
                                                     max_context_len))


def pa_prefill_chunk(query, key_cache, value_cache, block_tables, context_lens, cu_q_lens,
                     max_q_len, scale, max_context_len, out=None, workspace=None):
    """Causal chunk attention against the paged cache; returns float32 [total_q, Hq, d]."""
    dev = _dev(query, key_cache, value_cache, block_tables, context_lens, cu_q_lens)
    if cu_q_lens.dtype != torch.int32:
        raise TypeError("cu_q_lens must be int32")
    total_q, num_q_heads, head_dim = query.shape
    num_blocks, num_kv_heads, block_size, _ = key_cache.shape
    num_seqs = cu_q_lens.numel() - 1
    if out is None:
        out = torch.empty((total_q, num_q_heads, head_dim), dtype=torch.float32, device=dev)
    need = pa_prefill_chunk_workspace_size(num_seqs, total_q, max_q_len, num_q_heads,
                                           num_kv_heads, head_dim, block_size, max_context_len)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check("pa_prefill_chunk", lib().pa_prefill_chunk(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), _ptr(cu_q_lens), num_seqs, total_q, int(max_q_len), num_q_heads,
        num_kv_heads, head_dim, block_size, block_tables.shape[1], num_blocks,
        int(max_context_len), float(scale), _dtype_code(query), _ptr(workspace),
        workspace.numel() if workspace is not None else 0, _stream(dev)))
    return out


def pa_prefill_chunk_fp8(query, key_cache, value_cache, k_scale, v_scale, block_tables,
                         context_lens, cu_q_lens, max_q_len, scale, max_context_len, out=None,
                         workspace=None):
    """Causal chunk attention over an FP8 (E4M3) paged cache; returns float32
    [total_q, Hq, d]."""
    dev = _dev(query, key_cache, value_cache, k_scale, v_scale, block_tables, context_lens,
               cu_q_lens)
    if cu_q_lens.dtype != torch.int32:
        raise TypeError("cu_q_lens must be int32")
    _fp8_cache(key_cache)
    _fp8_cache(value_cache)
    _scales(k_scale, v_scale)
    total_q, num_q_heads, head_dim = query.shape
    num_blocks, num_kv_heads, block_size, _ = key_cache.shape
    if k_scale.numel() != num_kv_heads or v_scale.numel() != num_kv_heads:
        raise ValueError("one scale per KV head")
    num_seqs = cu_q_lens.numel() - 1
    if out is None:
        out = torch.empty((total_q, num_q_heads, head_dim), dtype=torch.float32, device=dev)
    need = pa_prefill_chunk_workspace_size(num_seqs, total_q, max_q_len, num_q_heads,
                                           num_kv_heads, head_dim, block_size, max_context_len)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check("pa_prefill_chunk_fp8", lib().pa_prefill_chunk_fp8(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_tables), _ptr(context_lens), _ptr(cu_q_lens), num_seqs, total_q,
        int(max_q_len), num_q_heads, num_kv_heads, head_dim, block_size, block_tables.shape[1],
        num_blocks, int(max_context_len), float(scale), _dtype_code(query), _ptr(workspace),
        workspace.numel() if workspace is not None else 0, _stream(dev)))
    return out


def pa_copy_blocks(key_cache, value_cache, pairs):
    """Copy block src to block dst of both caches for every row (src, dst) of
    the int64 [P, 2] device tensor ``pairs`` (pairs must be independent)."""
    dev = _dev(key_cache, value_cache, pairs)
    if pairs.dtype != torch.int64 or (pairs.numel() and pairs.shape[-1] != 2):
        raise TypeError("pairs must be int64 [num_pairs, 2]")
    if key_cache.dtype != value_cache.dtype:
        raise TypeError("key and value caches must share a dtype")
    num_blocks, num_kv_heads, block_size, head_dim = key_cache.shape
    _check("pa_copy_blocks", lib().pa_copy_blocks(
        _ptr(key_cache), _ptr(value_cache), _ptr(pairs), pairs.numel() // 2, num_kv_heads,
        head_dim, block_size, num_blocks, _dtype_code(key_cache), _stream(dev)))


def _swap(fn_name, key_cache, value_cache, host_key, host_value, pairs):
    dev = _dev(key_cache, value_cache)
    for t in (host_key, host_value):
        if t.device.type != "cpu" or not t.is_pinned() or not t.is_contiguous():
            raise ValueError("host pools must be contiguous pinned CPU tensors")
        if t.dtype != key_cache.dtype or t.shape[1:] != key_cache.shape[1:]:
            raise TypeError("host pools must match the caches' dtype and block shape")
    if pairs.dtype != torch.int64 or not pairs.is_contiguous() or \
            (pairs.numel() and pairs.shape[-1] != 2):
        raise TypeError("pairs must be contiguous int64 [num_pairs, 2]")
    if pairs.device.type == "cpu" and not pairs.is_pinned():
        raise ValueError("pairs must be on the GPU or in pinned host memory")
    num_blocks, num_kv_heads, block_size, head_dim = key_cache.shape
    _check(fn_name, getattr(lib(), fn_name)(
        _ptr(key_cache), _ptr(value_cache), _ptr(host_key), _ptr(host_value), _ptr(pairs),
        pairs.numel() // 2, num_kv_heads, head_dim, block_size, num_blocks, host_key.shape[0],
        _dtype_code(key_cache), _stream(dev)))


def pa_swap_out(key_cache, value_cache, host_key, host_value, pairs):
    """Copy device block b to host block h for every row (b, h) of pairs."""
    _swap("pa_swap_out", key_cache, value_cache, host_key, host_value, pairs)


def pa_swap_in(key_cache, value_cache, host_key, host_value, pairs):
    """Copy host block h to device block b for every row (h, b) of pairs."""
    _swap("pa_swap_in", key_cache, value_cache, host_key, host_value, pairs)


class BlockManager:
    """The host block manager of include/pa_blocks.h (C++ in libpa.so):
    on-demand blocks from a LIFO pool, reference-counted sharing by fork, and
    copy-on-write pairs for pa_copy_blocks. Not thread-safe."""

    def __init__(self, num_blocks, block_size, max_blocks_per_seq):
        self._lib = lib()
        h = _vp()
        _check("pa_bm_create", self._lib.pa_bm_create(num_blocks, block_size, max_blocks_per_seq,
                                                      ctypes.byref(h)))
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.max_blocks_per_seq = max_blocks_per_seq

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def add(self, seq):
        return self._lib.pa_bm_add(self._h, seq)

    def fork(self, parent, child):
        return self._lib.pa_bm_fork(self._h, parent, child)

    def append(self, seq, num_tokens):
        """(status, slots): slots is an int64 numpy array of num_tokens slots."""
        import numpy as np
        slots = np.empty(max(num_tokens, 0), dtype=np.int64)
        st = self._lib.pa_bm_append(self._h, seq, num_tokens, slots.ctypes.data_as(_vp))
        return st, (slots if st == 0 else slots[:0])

    def free(self, seq):
        return self._lib.pa_bm_free(self._h, seq)

    def num_free(self):
        return int(self._lib.pa_bm_num_free(self._h))

    def length(self, seq):
        return int(self._lib.pa_bm_length(self._h, seq))

    def blocks_needed(self, seq, num_tokens):
        return int(self._lib.pa_bm_blocks_needed(self._h, seq, num_tokens))

    def refcount(self, block):
        return int(self._lib.pa_bm_refcount(self._h, block))

    def table(self, seq):
        import numpy as np
        out = np.empty(self.max_blocks_per_seq, dtype=np.int32)
        n = self._lib.pa_bm_table(self._h, seq, out.ctypes.data_as(_vp), out.size)
        if n < 0:
            raise KeyError(seq)
        return out[:n].copy()

    def tables(self, seqs, row_stride=None):
        """(tables int32 [len(seqs), row_stride], context_lens int32) for one step."""
        import numpy as np
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        stride = row_stride or self.max_blocks_per_seq
        tables = np.empty((seqs.size, stride), dtype=np.int32)
        lens = np.empty(seqs.size, dtype=np.int32)
        _check("pa_bm_tables", self._lib.pa_bm_tables(
            self._h, seqs.ctypes.data_as(_vp), seqs.size, tables.ctypes.data_as(_vp), stride,
            lens.ctypes.data_as(_vp)))
        return tables, lens

    def take_copies(self, max_pairs=1 << 16):
        """One run of independent (src, dst) pairs as an int64 [P, 2] array."""
        import numpy as np
        pairs = np.empty((max_pairs, 2), dtype=np.int64)
        n = self._lib.pa_bm_take_copies(self._h, pairs.ctypes.data_as(_vp), max_pairs)
        return pairs[:n].copy()


class _SchedConfig(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int64), ("num_host_blocks", ctypes.c_int64),
                ("block_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("max_batch", ctypes.c_int32), ("chunk_tokens", ctypes.c_int32)]


_P64 = ctypes.POINTER(ctypes.c_int64)
_P32 = ctypes.POINTER(ctypes.c_int32)


class _StepPlan(ctypes.Structure):
    _fields_ = [("iteration", ctypes.c_int32),
                ("num_decode", ctypes.c_int32), ("decode_seqs", _P64), ("decode_slots", _P64),
                ("decode_context", _P32),
                ("num_prefill", ctypes.c_int32), ("prefill_seqs", _P64), ("prefill_start", _P32),
                ("prefill_cu", _P32), ("prefill_slots", _P64),
                ("num_swap_out", ctypes.c_int32), ("swap_out", _P64),
                ("num_swap_in", ctypes.c_int32), ("swap_in", _P64),
                ("num_finished", ctypes.c_int32), ("finished", _P64),
                ("num_admitted", ctypes.c_int32), ("admitted", _P64),
                ("num_preempted", ctypes.c_int32), ("preempted", _P64),
                ("num_resumed", ctypes.c_int32), ("resumed", _P64)]


class Scheduler:
    """The iteration-level batching scheduler of include/pa_sched.h (C++ in
    libpa.so) over an offline batch of (prompt_len, output_len) requests.
    ``step()`` returns the iteration's plan as numpy arrays."""

    def __init__(self, requests, *, num_blocks, num_host_blocks, block_size, max_blocks_per_seq,
                 max_batch, chunk_tokens):
        import numpy as np
        self._lib = lib()
        prompts = np.ascontiguousarray([int(p) for p, _ in requests], dtype=np.int32)
        outputs = np.ascontiguousarray([int(o) for _, o in requests], dtype=np.int32)
        cfg = _SchedConfig(num_blocks, num_host_blocks, block_size, max_blocks_per_seq, max_batch,
                           chunk_tokens)
        h = _vp()
        _check("pa_sched_create", self._lib.pa_sched_create(
            ctypes.byref(cfg), prompts.ctypes.data_as(_vp), outputs.ctypes.data_as(_vp),
            len(requests), ctypes.byref(h)))
        self._h = h
        self.block_size = block_size
        self.max_blocks_per_seq = max_blocks_per_seq
        self.requests = [(int(p), int(o)) for p, o in requests]

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pa_sched_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def done(self):
        return bool(self._lib.pa_sched_done(self._h))

    def step(self):
        plan = _StepPlan()
        _check("pa_sched_step", self._lib.pa_sched_step(self._h, ctypes.byref(plan)))
        return _plan_dict(plan)

    def tables(self, seqs, row_stride=None):
        """(tables int32 [len(seqs), row_stride], context_lens int32) of live sequences."""
        return _bm_tables(self._lib, self._lib.pa_sched_blocks(self._h), seqs,
                          row_stride or self.max_blocks_per_seq)


def _bm_tables(library, bm, seqs, stride):
    import numpy as np
    seqs = np.ascontiguousarray(seqs, dtype=np.int64)
    tables = np.empty((seqs.size, stride), dtype=np.int32)
    lens = np.empty(seqs.size, dtype=np.int32)
    _check("pa_bm_tables", library.pa_bm_tables(
        bm, seqs.ctypes.data_as(_vp), seqs.size, tables.ctypes.data_as(_vp), stride,
        lens.ctypes.data_as(_vp)))
    return tables, lens


def _plan_dict(plan):
    """A pa_step_plan as numpy arrays (copied)."""
    import numpy as np

    def arr(ptr, n, dtype):
        if n == 0:
            return np.zeros(0, dtype=dtype)
        return np.ctypeslib.as_array(ptr, shape=(n,)).astype(dtype, copy=True)

    npf = plan.num_prefill
    cu = arr(plan.prefill_cu, npf + 1, np.int32)
    return {
        "iteration": plan.iteration,
        "decode_seqs": arr(plan.decode_seqs, plan.num_decode, np.int64),
        "decode_slots": arr(plan.decode_slots, plan.num_decode, np.int64),
        "decode_context": arr(plan.decode_context, plan.num_decode, np.int32),
        "prefill_seqs": arr(plan.prefill_seqs, npf, np.int64),
        "prefill_start": arr(plan.prefill_start, npf, np.int32),
        "prefill_cu": cu,
        "prefill_slots": arr(plan.prefill_slots, int(cu[-1]), np.int64),
        "swap_out": arr(plan.swap_out, 2 * plan.num_swap_out, np.int64).reshape(-1, 2),
        "swap_in": arr(plan.swap_in, 2 * plan.num_swap_in, np.int64).reshape(-1, 2),
        "finished": arr(plan.finished, plan.num_finished, np.int64),
        "admitted": arr(plan.admitted, plan.num_admitted, np.int64),
        "preempted": arr(plan.preempted, plan.num_preempted, np.int64),
        "resumed": arr(plan.resumed, plan.num_resumed, np.int64),
    }

"""Thin ctypes binding of libpa (include/pa.h).

Argument marshalling only: every step runs in the HIP library.  Device memory
and the stream come from PyTorch (``tensor.data_ptr()``,
``torch.cuda.current_stream().cuda_stream``).  A missing library raises; there
is no fallback implementation.

Names follow the C entry points.  ``lib()`` exposes the raw C functions with
their ctypes signatures; the ``pa_*`` functions below take tensors.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PA_LIBRARY", os.path.join(HERE, "libpa.so"))

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP, PA_ERR_NO_BLOCKS = range(6)
PA_F32, PA_F16, PA_BF16 = 0, 1, 2

# Every symbol pa.h declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I32, _I64, _F32, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "pa_slot_mapping": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I32, _I32, _I64, _P]),
    "pa_reshape_and_cache": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I64, ctypes.c_int, _P]),
    "pa_decode_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "pa_decode_workspace_bytes_ex": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "pa_decode_attention": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                           _F32, ctypes.c_int, _P, _SZ, _P]),
    "pa_decode_attention_ex": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                              _F32, ctypes.c_int, _P, _SZ, _I32, _P]),
    "pa_decode_attention_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                                   _I32, _F32, ctypes.c_int, _I32, _P]),
    "pa_decode_partitions": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                            _F32, ctypes.c_int, _P, _SZ, _I32, _P]),
    "pa_decode_combine": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _I32, _I32, ctypes.c_int, _P, _SZ, _P]),
    "pa_decode_partition_size": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32, ctypes.c_int, _P]),
    "pa_decode_plan_partition_size": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32, ctypes.c_int, _P, _I32, _I32]),
    "pa_prefill_attention": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                            _I32, _I32, _F32, ctypes.c_int, _P, _SZ, _I32, _P]),
    "pa_prefill_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "pa_copy_blocks": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I32, _I32, _I32, _I64, ctypes.c_int, _P]),
    "pa_swap_blocks": (ctypes.c_int, [_P, _P, _I64, _P, _P, _I64, _P, _P, _I64, _I32, _I32, _I32, ctypes.c_int, _P]),
    "pa_block_pool_create": (_P, [_I32, _I32, _P]),
    "pa_block_pool_destroy": (None, [_P]),
    "pa_block_pool_num_free": (_I32, [_P]),
    "pa_block_pool_ref_count": (_I32, [_P, _I32]),
    "pa_block_pool_allocate": (ctypes.c_int, [_P, _I32, _P]),
    "pa_block_pool_free": (ctypes.c_int, [_P, _P, _I32]),
    "pa_seq_create": (ctypes.c_int, [_P, _P]),
    "pa_seq_fork": (ctypes.c_int, [_P, _I32, _P]),
    "pa_seq_append": (ctypes.c_int, [_P, _I32, _I64, _P, _P]),
    "pa_seq_release": (ctypes.c_int, [_P, _I32]),
    "pa_seq_length": (_I64, [_P, _I32]),
    "pa_seq_block_table": (ctypes.c_int, [_P, _I32, _P, _I32, _P]),
    "pa_decode_attention_shared_prefix": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32,
                                                         _I32, _I32, _I32, _I32, _I32, _I32, _F32, ctypes.c_int,
                                                         _P, _SZ, _P]),
    "pa_decode_attention_shared_prefix_layout": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32,
                                                                _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                                                _F32, ctypes.c_int, _P, _SZ, ctypes.c_int, _P]),
    "pa_shared_prefix_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "pa_shared_prefix_groups": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P]),
    "pa_reshape_and_cache_layout": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I64, ctypes.c_int,
                                                   ctypes.c_int, _P]),
    "pa_decode_attention_layout": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                                  _F32, ctypes.c_int, _P, _SZ, _I32, ctypes.c_int, _P]),
    "pa_prefill_attention_layout": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                                   _I32, _I32, _I32, _F32, ctypes.c_int, _P, _SZ, _I32,
                                                   ctypes.c_int, _P]),
    "pa_convert_blocks": (ctypes.c_int, [_P, _P, ctypes.c_int, _I64, _P, _P, ctypes.c_int, _I64, _P, _P, _I64, _I32,
                                         _I32, _I32, ctypes.c_int, _P]),
    "pa_write_new_tokens": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I64,
                                           ctypes.c_int, ctypes.c_int, _P]),
    "pa_decode_step": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I64,
                                      _I32, _F32, ctypes.c_int, _P, _SZ, _I32, ctypes.c_int, _P]),
    "pa_stream_read": (ctypes.c_int, [_P, _SZ, _P, ctypes.c_int, _P]),
    "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}

_LIB = None


def lib():
    """Load libpa.so (once) and attach the C signatures."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libpa not built: {LIB_PATH} is missing "
                               "(run `python -m paged_kv_cache_size_amd.build`)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def pa_status_string(status: int) -> str:
    return lib().pa_status_string(int(status)).decode()


class PAError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {pa_status_string(status)}")
        self.status = status


def _check(rc: int, where: str):
    if rc != PA_OK:
        raise PAError(rc, where)


# --------------------------------------------------------------------- tensors

def _torch():
    import torch
    return torch


def pa_dtype(t) -> int:
    torch = _torch()
    m = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _dev(t, name, dtype=None, ndim=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


PA_KV_SPLIT, PA_KV_FUSED = 0, 1  # pa_kv_layout


def _pool(k_pool, v_pool, layout, host_ok=False):
    """(num_blocks, block_size, num_kv_heads, head_dim) of a pool in
    ``layout`` and its two C pointers (the second None for the fused pool
    [NB, H_kv, BS, 2D], passed as ``k_pool`` with ``v_pool=None``)."""
    check = _host_or_dev if host_ok else _dev
    if layout == PA_KV_SPLIT:
        if v_pool is None or v_pool.shape != k_pool.shape or v_pool.dtype != k_pool.dtype:
            raise ValueError("the split layout takes a K and a V pool of one shape and dtype")
        nb, bs, hkv, d = k_pool.shape
        return (nb, bs, hkv, d), check(k_pool, "k_pool", ndim=4), check(v_pool, "v_pool", ndim=4)
    if layout == PA_KV_FUSED:
        if v_pool is not None:
            raise ValueError("the fused layout takes one pool [NB, H_kv, BS, 2D] (v_pool=None)")
        nb, hkv, bs, d2 = k_pool.shape
        if d2 % 2:
            raise ValueError("a fused pool's last axis holds K and V: 2 * head_dim")
        return (nb, bs, hkv, d2 // 2), check(k_pool, "kv_pool", ndim=4), None
    raise ValueError(f"unknown layout {layout}")


def _host_or_dev(t, name, ndim=None):
    """Pointer of a contiguous device tensor or pinned host tensor."""
    if not t.is_contiguous() or not (t.is_cuda or t.is_pinned()):
        raise ValueError(f"{name} must be a contiguous device tensor or pinned host tensor")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def pa_slot_mapping(block_tables, context_lens, block_size: int, query_start_loc=None,
                    num_tokens: int | None = None, out=None):
    """int64 slot of every new token (see pa.h).  Decode when
    ``query_start_loc`` is None; otherwise ``num_tokens`` (host int) is
    required."""
    torch = _torch()
    B, mb = block_tables.shape
    if query_start_loc is None:
        num_tokens = B
    elif num_tokens is None:
        raise ValueError("num_tokens is required with query_start_loc")
    if out is None:
        out = torch.empty(num_tokens, dtype=torch.int64, device=block_tables.device)
    rc = lib().pa_slot_mapping(
        _dev(out, "out", torch.int64, 1), _dev(block_tables, "block_tables", torch.int32, 2),
        _dev(context_lens, "context_lens", torch.int32, 1),
        None if query_start_loc is None else _dev(query_start_loc, "query_start_loc", torch.int32, 1),
        B, mb, int(block_size), int(num_tokens), _stream(block_tables))
    _check(rc, "pa_slot_mapping")
    return out


def pa_reshape_and_cache(key, value, k_pool, v_pool, slot_mapping, layout: int = PA_KV_SPLIT):
    """Write key/value rows [N, H_kv, D] into the pools at slot_mapping
    (``layout`` PA_KV_FUSED: ``k_pool`` is the fused pool, ``v_pool`` None)."""
    torch = _torch()
    (nb, bs, hkv, d), kp, vp = _pool(k_pool, v_pool, layout)
    if key.shape != value.shape:
        raise ValueError("key/value shapes must match")
    if not (key.dtype == value.dtype == k_pool.dtype):
        raise TypeError("key, value and pools must share a dtype")
    if tuple(key.shape[1:]) != (hkv, d):
        raise ValueError(f"key rows {tuple(key.shape[1:])} do not match pool rows {(hkv, d)}")
    n = key.shape[0]
    if slot_mapping.shape != (n,):
        raise ValueError("slot_mapping must be [num_tokens]")
    args = (_dev(key, "key", ndim=3), _dev(value, "value", ndim=3), kp, vp,
            _dev(slot_mapping, "slot_mapping", torch.int64, 1), n, hkv, d, bs, nb, pa_dtype(key))
    if layout == PA_KV_SPLIT:
        rc = lib().pa_reshape_and_cache(*args, _stream(key))
    else:
        rc = lib().pa_reshape_and_cache_layout(*args, int(layout), _stream(key))
    _check(rc, "pa_reshape_and_cache")


def pa_write_new_tokens(key, value, k_pool, v_pool, block_tables, context_lens, slot_out=None,
                        layout: int = PA_KV_SPLIT):
    """Slot mapping and pool write of a decode step in one launch: each
    sequence's new token (its last context position) into its slot; the
    slots go to ``slot_out`` (int64 [B]) when given (see pa.h)."""
    torch = _torch()
    (nb, bs, hkv, d), kp, vp = _pool(k_pool, v_pool, layout)
    B = block_tables.shape[0]
    if key.shape != (B, hkv, d) or value.shape != key.shape:
        raise ValueError(f"key/value must be [num_seqs, num_kv_heads, head_dim] = {(B, hkv, d)}")
    if not (key.dtype == value.dtype == k_pool.dtype):
        raise TypeError("key, value and pools must share a dtype")
    if context_lens.shape != (B,):
        raise ValueError("context_lens must be [num_seqs]")
    rc = lib().pa_write_new_tokens(
        _dev(key, "key", ndim=3), _dev(value, "value", ndim=3), kp, vp,
        _dev(block_tables, "block_tables", torch.int32, 2), _dev(context_lens, "context_lens", torch.int32, 1),
        None if slot_out is None else _dev(slot_out, "slot_out", torch.int64, 1), B, hkv, d, bs,
        block_tables.shape[1], nb, pa_dtype(key), int(layout), _stream(key))
    _check(rc, "pa_write_new_tokens")
    return slot_out


def pa_decode_step(query, key, value, k_pool, v_pool, block_tables, context_lens, scale: float,
                   max_context_len: int, out=None, workspace=None, slot_out=None, partition_size: int = 0,
                   layout: int = PA_KV_SPLIT):
    """A whole decode step in one library call: the new tokens' slots and
    K/V rows (one launch), then paged attention over the contexts that
    include them; returns ``out`` [B, H, D] (see pa.h)."""
    torch = _torch()
    B, H, D = query.shape
    (nb, bs, hkv, d2), kp, vp = _pool(k_pool, v_pool, layout)
    if d2 != D or key.shape != (B, hkv, D) or value.shape != key.shape:
        raise ValueError("query / key / value / pool shapes do not match")
    if not (query.dtype == key.dtype == value.dtype == k_pool.dtype):
        raise TypeError("query, key, value and pools must share a dtype")
    if block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables / context_lens batch mismatch")
    if out is None:
        out = torch.empty_like(query)
    need = pa_decode_workspace_bytes(B, H, D, max_context_len, bs, partition_size)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_ptr = None if workspace is None else _dev(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().pa_decode_step(
        _dev(out, "out", query.dtype, 3), _dev(query, "query", ndim=3), _dev(key, "key", ndim=3),
        _dev(value, "value", ndim=3), kp, vp, _dev(block_tables, "block_tables", torch.int32, 2),
        _dev(context_lens, "context_lens", torch.int32, 1),
        None if slot_out is None else _dev(slot_out, "slot_out", torch.int64, 1), B, H, hkv, D, bs,
        block_tables.shape[1], nb, int(max_context_len), float(scale), pa_dtype(query), ws_ptr, ws_bytes,
        int(partition_size), int(layout), _stream(query))
    _check(rc, "pa_decode_step")
    return out


def pa_decode_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len, block_size,
                              partition_size: int = 0) -> int:
    return int(lib().pa_decode_workspace_bytes_ex(num_seqs, num_heads, head_dim, max_context_len,
                                                  block_size, partition_size))


def _host_lens(context_lens, num_seqs):
    """Host int32 copy of the context lengths (kept alive by the caller) and
    its pointer, or (None, None)."""
    if context_lens is None:
        return None, None
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32).reshape(-1))
    if arr.shape[0] != num_seqs:
        raise ValueError(f"context_lens has {arr.shape[0]} entries, num_seqs is {num_seqs}")
    return arr, ctypes.c_void_p(arr.ctypes.data)


def _dtype_code(dtype) -> int:
    return dtype if isinstance(dtype, int) else pa_dtype(_torch().empty(0, dtype=dtype))


def pa_decode_partition_size(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, block_size,
                             dtype, context_lens=None) -> int:
    """``dtype``: a torch dtype or a PA_* code; ``context_lens``: None or the
    host-side lengths (a sequence of ints / numpy array)."""
    arr, ptr = _host_lens(context_lens, num_seqs)
    ps = int(lib().pa_decode_partition_size(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len,
                                            block_size, _dtype_code(dtype), ptr))
    del arr
    if ps < 0:
        raise PAError(-ps, "pa_decode_partition_size")
    return ps


def pa_decode_plan_partition_size(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, block_size,
                                  dtype, context_lens, num_cus, workgroups_per_cu) -> int:
    """Device-free form of pa_decode_partition_size for a given geometry."""
    arr, ptr = _host_lens(context_lens, num_seqs)
    ps = int(lib().pa_decode_plan_partition_size(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len,
                                                 block_size, _dtype_code(dtype), ptr, num_cus,
                                                 workgroups_per_cu))
    del arr
    if ps < 0:
        raise PAError(-ps, "pa_decode_plan_partition_size")
    return ps


def pa_decode_attention(query, k_pool, v_pool, block_tables, context_lens, scale: float,
                        max_context_len: int | None = None, out=None, workspace=None,
                        partition_size: int = 0, layout: int = PA_KV_SPLIT):
    """One decode step of paged attention; returns ``out`` [B, H, D].

    ``max_context_len`` is a host int bounding context_lens (reading it from
    the device would synchronise; pass it when known).  The workspace is
    allocated with PyTorch when not given.  ``layout`` PA_KV_FUSED: ``k_pool``
    is the fused pool and ``v_pool`` None."""
    torch = _torch()
    B, H, D = query.shape
    (nb, bs, hkv, d2), kp, vp = _pool(k_pool, v_pool, layout)
    if d2 != D:
        raise ValueError("pool shape does not match query")
    if query.dtype != k_pool.dtype:
        raise TypeError("query and pools must share a dtype")
    if block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables / context_lens batch mismatch")
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if B else 0
    mb = block_tables.shape[1]
    if out is None:
        out = torch.empty_like(query)
    need = pa_decode_workspace_bytes(B, H, D, max_context_len, bs, partition_size)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_ptr = None if workspace is None else _dev(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_dev(out, "out", query.dtype, 3), _dev(query, "query", ndim=3), kp, vp,
            _dev(block_tables, "block_tables", torch.int32, 2), _dev(context_lens, "context_lens", torch.int32, 1),
            B, H, hkv, D, bs, mb, int(max_context_len), float(scale), pa_dtype(query), ws_ptr, ws_bytes,
            int(partition_size))
    if layout == PA_KV_SPLIT:
        rc = lib().pa_decode_attention_ex(*args, _stream(query))
    else:
        rc = lib().pa_decode_attention_layout(*args, int(layout), _stream(query))
    _check(rc, "pa_decode_attention")
    return out


def pa_prefill_workspace_bytes(num_tokens, num_heads, head_dim, max_context_len, block_size,
                               partition_size: int = 0) -> int:
    return int(lib().pa_prefill_workspace_bytes(num_tokens, num_heads, head_dim, max_context_len, block_size,
                                                partition_size))


def pa_prefill_attention(query, k_pool, v_pool, block_tables, context_lens, query_start_loc, scale: float,
                         max_query_len: int, max_context_len: int, out=None, workspace=None,
                         partition_size: int = 0, layout: int = PA_KV_SPLIT):
    """Paged attention of several new tokens per sequence; returns ``out`` [T, H, D].

    ``query_start_loc`` (int32 [B+1], device) delimits each sequence's rows of
    ``query``; ``context_lens`` include the new tokens, whose K/V must already
    be in the pools.  ``max_query_len`` / ``max_context_len`` are host bounds.
    ``layout`` PA_KV_FUSED: ``k_pool`` is the fused pool and ``v_pool`` None."""
    torch = _torch()
    T, H, D = query.shape
    (nb, bs, hkv, d2), kp, vp = _pool(k_pool, v_pool, layout)
    B = block_tables.shape[0]
    if d2 != D:
        raise ValueError("pool shape does not match query")
    if query.dtype != k_pool.dtype:
        raise TypeError("query and pools must share a dtype")
    if context_lens.shape != (B,) or query_start_loc.shape != (B + 1,):
        raise ValueError("context_lens / query_start_loc do not match the block tables' batch")
    if out is None:
        out = torch.empty_like(query)
    need = pa_prefill_workspace_bytes(T, H, D, int(max_context_len), bs, partition_size)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_ptr = None if workspace is None else _dev(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_dev(out, "out", query.dtype, 3), _dev(query, "query", ndim=3), kp, vp,
            _dev(block_tables, "block_tables", torch.int32, 2), _dev(context_lens, "context_lens", torch.int32, 1),
            _dev(query_start_loc, "query_start_loc", torch.int32, 1), B, T, int(max_query_len), H, hkv, D, bs,
            block_tables.shape[1], int(max_context_len), float(scale), pa_dtype(query), ws_ptr, ws_bytes,
            int(partition_size))
    if layout == PA_KV_SPLIT:
        rc = lib().pa_prefill_attention(*args, _stream(query))
    else:
        rc = lib().pa_prefill_attention_layout(*args, int(layout), _stream(query))
    _check(rc, "pa_prefill_attention")
    return out


def pa_copy_blocks(k_pool, v_pool, src_blocks, dst_blocks):
    """Copy whole blocks src -> dst in both pools (int64 device id tensors)."""
    torch = _torch()
    nb, bs, hkv, d = k_pool.shape
    if v_pool.shape != k_pool.shape or v_pool.dtype != k_pool.dtype:
        raise ValueError("k_pool and v_pool differ")
    n = int(src_blocks.numel())
    if dst_blocks.numel() != n:
        raise ValueError("src_blocks and dst_blocks differ in length")
    rc = lib().pa_copy_blocks(_dev(k_pool, "k_pool", ndim=4), _dev(v_pool, "v_pool", ndim=4),
                              _dev(src_blocks, "src_blocks", torch.int64, 1) if n else None,
                              _dev(dst_blocks, "dst_blocks", torch.int64, 1) if n else None, n, bs, hkv, d, nb,
                              pa_dtype(k_pool), _stream(k_pool))
    _check(rc, "pa_copy_blocks")


def pa_swap_blocks(dst_k_pool, dst_v_pool, src_k_pool, src_v_pool, src_blocks, dst_blocks, stream_of=None):
    """Copy whole blocks src pools -> dst pools (either pair may be pinned
    host tensors); id tensors (int64) on the device."""
    torch = _torch()
    if dst_k_pool.shape[1:] != src_k_pool.shape[1:] or dst_k_pool.dtype != src_k_pool.dtype:
        raise ValueError("pools differ in block shape or dtype")
    for t in (dst_k_pool, dst_v_pool, src_k_pool, src_v_pool):
        if not t.is_contiguous() or not (t.is_cuda or t.is_pinned()):
            raise ValueError("pools must be contiguous device tensors or pinned host tensors")
    n = int(src_blocks.numel())
    if dst_blocks.numel() != n:
        raise ValueError("src_blocks and dst_blocks differ in length")
    _, bs, hkv, d = dst_k_pool.shape
    dev = stream_of if stream_of is not None else (src_blocks if n else dst_k_pool)
    rc = lib().pa_swap_blocks(
        ctypes.c_void_p(dst_k_pool.data_ptr()), ctypes.c_void_p(dst_v_pool.data_ptr()), dst_k_pool.shape[0],
        ctypes.c_void_p(src_k_pool.data_ptr()), ctypes.c_void_p(src_v_pool.data_ptr()), src_k_pool.shape[0],
        _dev(src_blocks, "src_blocks", torch.int64, 1) if n else None,
        _dev(dst_blocks, "dst_blocks", torch.int64, 1) if n else None, n, bs, hkv, d, pa_dtype(dst_k_pool),
        _stream(dev) if dev.is_cuda else None)
    _check(rc, "pa_swap_blocks")


def pa_convert_blocks(dst_k, dst_v, dst_layout: int, src_k, src_v, src_layout: int, src_blocks, dst_blocks):
    """Copy whole blocks between pools of any layouts (either may be pinned
    host tensors); id tensors int64 on the device."""
    torch = _torch()
    dshape, dk, dv = _pool(dst_k, dst_v, dst_layout, host_ok=True)
    sshape, sk, sv = _pool(src_k, src_v, src_layout, host_ok=True)
    if dshape[1:] != sshape[1:] or dst_k.dtype != src_k.dtype:
        raise ValueError("pools differ in block shape or dtype")
    n = int(src_blocks.numel())
    if dst_blocks.numel() != n:
        raise ValueError("src_blocks and dst_blocks differ in length")
    _, bs, hkv, d = dshape
    dev = src_blocks if n else (dst_k if dst_k.is_cuda else src_k)
    rc = lib().pa_convert_blocks(
        dk, dv, int(dst_layout), dshape[0], sk, sv, int(src_layout), sshape[0],
        _dev(src_blocks, "src_blocks", torch.int64, 1) if n else None,
        _dev(dst_blocks, "dst_blocks", torch.int64, 1) if n else None, n, bs, hkv, d, pa_dtype(dst_k),
        _stream(dev) if dev.is_cuda else None)
    _check(rc, "pa_convert_blocks")


def pa_stream_read(buf, sink, nontemporal: bool = False):
    """Read every byte of the device tensor ``buf`` once (a measurement of
    the device's streaming read rate); ``sink`` is a device int32 tensor."""
    _dev(buf, "buf")
    _dev(sink, "sink", _torch().int32)
    nbytes = buf.numel() * buf.element_size()
    rc = lib().pa_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                              int(bool(nontemporal)), _stream(buf))
    _check(rc, "pa_stream_read")


class SharedPrefixGroups:
    """Groups of consecutive sequences sharing leading blocks (host arrays)."""

    def __init__(self, group_start, prefix_lens, seq_prefix_lens, max_group_size, max_prefix_len):
        self.group_start, self.prefix_lens, self.seq_prefix_lens = group_start, prefix_lens, seq_prefix_lens
        self.max_group_size, self.max_prefix_len = int(max_group_size), int(max_prefix_len)

    @property
    def num_groups(self) -> int:
        return int(self.prefix_lens.shape[0])


def pa_shared_prefix_groups(block_tables, context_lens, block_size: int, min_prefix_blocks: int = 1):
    """Find the shared-prefix groups from host (numpy) tables and lengths."""
    import numpy as np
    bt = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    B, mb = bt.shape
    gs = np.zeros(B + 1, np.int32)
    pl = np.zeros(B, np.int32)
    spl = np.zeros(B, np.int32)
    ng, gmax, pmax = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    p = lambda a: ctypes.c_void_p(a.ctypes.data)  # noqa: E731
    rc = lib().pa_shared_prefix_groups(p(bt), p(lens), B, mb, int(block_size), int(min_prefix_blocks), p(gs), p(pl),
                                       p(spl), ctypes.byref(ng), ctypes.byref(gmax), ctypes.byref(pmax))
    _check(rc, "pa_shared_prefix_groups")
    n = ng.value
    return SharedPrefixGroups(gs[:n + 1].copy(), pl[:n].copy(), spl, gmax.value, pmax.value)


def pa_decode_attention_shared_prefix(query, k_pool, v_pool, block_tables, context_lens, groups, scale: float,
                                      max_context_len: int, out=None, workspace=None, device_groups=None,
                                      layout: int = PA_KV_SPLIT):
    """Cascade decode: shared prefixes read once per group.  ``groups`` is a
    SharedPrefixGroups; ``device_groups`` optionally its three arrays already
    on the device (group_start, prefix_lens, seq_prefix_lens).  ``layout``
    PA_KV_FUSED: ``k_pool`` is the fused pool and ``v_pool`` None."""
    torch = _torch()
    B, H, D = query.shape
    (nb, bs, hkv, d2), kp, vp = _pool(k_pool, v_pool, layout)
    if d2 != D or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("shapes do not match")
    if device_groups is None:
        device_groups = tuple(torch.from_numpy(x).to(query.device)
                              for x in (groups.group_start, groups.prefix_lens, groups.seq_prefix_lens))
    gs, pl, spl = device_groups
    if out is None:
        out = torch.empty_like(query)
    need = int(lib().pa_shared_prefix_workspace_bytes(B, H, D, int(max_context_len), groups.max_prefix_len))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=query.device)
    args = (_dev(out, "out", query.dtype, 3), _dev(query, "query", ndim=3), kp, vp,
            _dev(block_tables, "block_tables", torch.int32, 2), _dev(context_lens, "context_lens", torch.int32, 1),
            _dev(gs, "group_start", torch.int32, 1), _dev(pl, "prefix_lens", torch.int32, 1),
            _dev(spl, "seq_prefix_lens", torch.int32, 1), B, groups.num_groups, groups.max_group_size, H, hkv, D, bs,
            block_tables.shape[1], int(max_context_len), groups.max_prefix_len, float(scale), pa_dtype(query),
            _dev(workspace, "workspace"), workspace.numel() * workspace.element_size())
    if layout == PA_KV_SPLIT:
        rc = lib().pa_decode_attention_shared_prefix(*args, _stream(query))
    else:
        rc = lib().pa_decode_attention_shared_prefix_layout(*args, int(layout), _stream(query))
    _check(rc, "pa_decode_attention_shared_prefix")
    return out


class BlockManager:
    """The library's host block pool and its sequences (pa_block_pool_*, pa_seq_*)."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self._order = None
        ptr = None
        if free_order is not None:
            import numpy as np
            self._order = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
            if self._order.shape != (num_blocks,):
                raise ValueError("free_order must list every block once")
            ptr = ctypes.c_void_p(self._order.ctypes.data)
        self._lib = lib()
        self._h = self._lib.pa_block_pool_create(int(num_blocks), int(block_size), ptr)
        if not self._h:
            raise PAError(PA_ERR_INVALID_ARG, "pa_block_pool_create")
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pa_block_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def num_free(self) -> int:
        return int(self._lib.pa_block_pool_num_free(self._h))

    def ref_count(self, block: int) -> int:
        return int(self._lib.pa_block_pool_ref_count(self._h, int(block)))

    def allocate(self, n: int):
        """n block ids, or None when the pool is short (nothing changes)."""
        buf = (ctypes.c_int32 * max(int(n), 1))()
        rc = self._lib.pa_block_pool_allocate(self._h, int(n), buf)
        if rc == PA_ERR_NO_BLOCKS:
            return None
        _check(rc, "pa_block_pool_allocate")
        return list(buf[:n])

    def free(self, blocks) -> None:
        arr = (ctypes.c_int32 * max(len(blocks), 1))(*[int(b) for b in blocks])
        _check(self._lib.pa_block_pool_free(self._h, arr, len(blocks)), "pa_block_pool_free")

    def new_seq(self) -> int:
        h = ctypes.c_int32()
        _check(self._lib.pa_seq_create(self._h, ctypes.byref(h)), "pa_seq_create")
        return h.value

    def fork(self, seq: int) -> int:
        h = ctypes.c_int32()
        _check(self._lib.pa_seq_fork(self._h, int(seq), ctypes.byref(h)), "pa_seq_fork")
        return h.value

    def append(self, seq: int, num_tokens: int):
        """Grow a sequence; returns the copy-on-write pair (src, dst) or None."""
        src, dst = ctypes.c_int32(), ctypes.c_int32()
        _check(self._lib.pa_seq_append(self._h, int(seq), int(num_tokens), ctypes.byref(src), ctypes.byref(dst)),
               "pa_seq_append")
        return None if src.value < 0 else (src.value, dst.value)

    def release(self, seq: int) -> None:
        _check(self._lib.pa_seq_release(self._h, int(seq)), "pa_seq_release")

    def length(self, seq: int) -> int:
        return int(self._lib.pa_seq_length(self._h, int(seq)))

    def block_table(self, seq: int):
        n = ctypes.c_int32()
        rc = self._lib.pa_seq_block_table(self._h, int(seq), None, 0, ctypes.byref(n))
        if rc not in (PA_OK, PA_ERR_WORKSPACE):
            _check(rc, "pa_seq_block_table")
        buf = (ctypes.c_int32 * max(n.value, 1))()
        _check(self._lib.pa_seq_block_table(self._h, int(seq), buf, n.value, ctypes.byref(n)), "pa_seq_block_table")
        return list(buf[:n.value])


def _decode_common(query, k_pool, v_pool, block_tables, context_lens, out):
    torch = _torch()
    B, H, D = query.shape
    nb, bs, hkv, d2 = k_pool.shape
    if d2 != D or k_pool.shape != v_pool.shape:
        raise ValueError("pool shape does not match query")
    if not (query.dtype == k_pool.dtype == v_pool.dtype):
        raise TypeError("query and pools must share a dtype")
    if block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables / context_lens batch mismatch")
    if out is None:
        out = torch.empty_like(query)
    return B, H, D, bs, hkv, out


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()


def pa_decode_partitions(query, k_pool, v_pool, block_tables, context_lens, scale: float,
                         max_context_len: int, partition_size: int, workspace=None, out=None):
    """Stage 1 of decode attention (see pa.h); ``partition_size`` explicit."""
    torch = _torch()
    B, H, D, bs, hkv, out = _decode_common(query, k_pool, v_pool, block_tables, context_lens, out)
    ws_ptr, ws_bytes = _ws(workspace)
    rc = lib().pa_decode_partitions(
        _dev(out, "out", query.dtype, 3), _dev(query, "query", ndim=3), _dev(k_pool, "k_pool", ndim=4),
        _dev(v_pool, "v_pool", ndim=4), _dev(block_tables, "block_tables", torch.int32, 2),
        _dev(context_lens, "context_lens", torch.int32, 1), B, H, hkv, D, bs, block_tables.shape[1],
        int(max_context_len), float(scale), pa_dtype(query), ws_ptr, ws_bytes, int(partition_size),
        _stream(query))
    _check(rc, "pa_decode_partitions")
    return out


def pa_decode_combine(out, context_lens, max_context_len: int, partition_size: int, workspace=None):
    """Stage 2 of decode attention: merge partition partials into ``out``."""
    torch = _torch()
    B, H, D = out.shape
    ws_ptr, ws_bytes = _ws(workspace)
    rc = lib().pa_decode_combine(
        _dev(out, "out", ndim=3), _dev(context_lens, "context_lens", torch.int32, 1), B, H, D,
        int(max_context_len), int(partition_size), pa_dtype(out), ws_ptr, ws_bytes, _stream(out))
    _check(rc, "pa_decode_combine")
    return out


def decode_step(query, key, value, k_pool, v_pool, block_tables, context_lens, scale: float,
                max_context_len: int, out=None, workspace=None, slot_out=None, partition_size: int = 0):
    """The whole decode hot path on one stream: slots of the new tokens,
    their K/V written into the pools, then paged attention (pa_decode_step)."""
    return pa_decode_step(query, key, value, k_pool, v_pool, block_tables, context_lens, scale, max_context_len,
                          out=out, workspace=workspace, slot_out=slot_out, partition_size=partition_size)

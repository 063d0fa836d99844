"""ctypes binding of libpa.so: argument marshalling only.

Every function here forwards to the C entry point of the same name declared in
``include/pa.h``.  Device arrays are passed as torch tensors (their data
pointers go across the ABI); host arrays of the block manager as NumPy arrays.
No computation of the method happens in Python: there is no fallback, and a
missing library raises at import of this module.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PA_LIBRARY", os.path.join(_HERE, "libpa.so"))
# PA_HOST_ONLY=1: LIB_PATH is a host-only build of the block manager
# (libpa_host.so, libpa_host_asan.so): torch is not loaded and only the pa_bm_*
# entry points and the status strings are bound.
HOST_ONLY = os.environ.get("PA_HOST_ONLY", "") == "1"

PA_OK = 0
PA_ERR_INVALID_ARG = 1
PA_ERR_UNSUPPORTED = 2
PA_ERR_NO_FREE_BLOCKS = 3
PA_ERR_EXISTS = 4
PA_ERR_NOT_FOUND = 5
PA_ERR_WORKSPACE = 6
PA_ERR_HIP = 7
PA_F32 = 0
PA_BF16 = 1
PA_FP8_E4M3 = 2
PA_INT8 = 3

# torch first: libpa.so then binds to the HIP runtime torch has loaded, so
# torch's streams and device memory are valid in the library's calls.
if not HOST_ONLY:
    import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libpa.so not found at {LIB_PATH}; build it with "
                      f"`python paged_kv_cache_124_amd/build.py`")
lib = ctypes.CDLL(LIB_PATH)


class PAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib.pa_status_string(status).decode()} (status {status})")


class BMCacheStats(ctypes.Structure):
    _fields_ = [(n, c_int64) for n in ("enabled", "num_cached", "num_idle", "hit_blocks", "evictions")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


class BMStats(ctypes.Structure):
    _fields_ = [(n, c_int64) for n in ("num_blocks", "num_free", "num_used", "num_seqs",
                                       "cow_copies", "stored_tokens", "tail_waste_slots")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


_P32 = POINTER(c_int32)
_P64 = POINTER(c_int64)
_SIGS = {
    "pa_status_string": (ctypes.c_char_p, [c_int]),
    "pa_version": (c_int, []),
    "pa_decode": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int,
                          c_int, c_float, c_int, c_int, c_int, c_int, c_void_p, c_size_t, c_void_p]),
    "pa_decode_step": (c_int, [c_void_p] * 9 + [c_int] * 5 + [c_float] + [c_int] * 4 + [c_void_p, c_size_t, c_void_p]),
    "pa_decode_workspace_bytes": (c_size_t, [c_int] * 7),
    "pa_decode_step_noalloc": (c_int, [c_void_p] * 9 + [c_int] * 5 + [c_float] + [c_int] * 4 + [c_void_p]),
    "pa_decode_partitioned": (c_int, [c_void_p] * 6 + [c_int] * 5 + [c_float] + [c_int] * 5
                              + [c_void_p, c_size_t, c_void_p]),
    "pa_decode_partitioned_workspace_bytes": (c_size_t, [c_int] * 8),
    "pa_check_batch": (c_int, [c_void_p, c_void_p] + [c_int] * 5 + [c_void_p, c_void_p]),
    "pa_check_pairs": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p]),
    "pa_decode_shared": (c_int, [c_void_p] * 7 + [c_int] * 6 + [c_float] + [c_int] * 4 + [c_void_p, c_size_t, c_void_p]),
    "pa_decode_step_shared": (c_int, [c_void_p] * 10 + [c_int] * 6 + [c_float] + [c_int] * 4
                              + [c_void_p, c_size_t, c_void_p]),
    "pa_decode_shared_workspace_bytes": (c_size_t, [c_int] * 8),
    "pa_decode_partition_tokens": (c_int, [c_int] * 7),
    "pa_append_kv": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int,
                             c_int, c_void_p]),
    "pa_append_step": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int,
                               c_int, c_int, c_int, c_int, c_int, c_void_p]),
    "pa_copy_blocks": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int, c_int, c_int64,
                               c_int, c_void_p]),
    "pa_decode_fp8": (c_int, [c_void_p] * 7 + [c_int] * 5 + [c_float] + [c_int] * 3 + [c_void_p, c_size_t, c_void_p]),
    "pa_append_kv_fp8": (c_int, [c_void_p] * 6 + [c_int] * 5 + [c_void_p]),
    "pa_copy_blocks_fp8": (c_int, [c_void_p] * 4 + [c_int] * 6 + [c_int64, c_int64, c_void_p]),
    "pa_append_step_fp8": (c_int, [c_void_p] * 8 + [c_int] * 6 + [c_void_p]),
    "pa_swap_blocks": (c_int, [c_void_p] * 5 + [c_int] * 8 + [c_int64, c_int64, c_void_p]),
    "pa_swap_blocks_fp8": (c_int, [c_void_p] * 7 + [c_int] * 6 + [c_int64] * 4 + [c_void_p]),
    "pa_decode_step_fp8": (c_int, [c_void_p] * 10 + [c_int] * 5 + [c_float] + [c_int] * 3 +
                           [c_void_p, c_size_t, c_void_p]),
    "pa_decode_step_int8": (c_int, [c_void_p] * 10 + [c_int] * 5 + [c_float] + [c_int] * 3 +
                            [c_void_p, c_size_t, c_void_p]),
    "pa_decode_int8": (c_int, [c_void_p] * 7 + [c_int] * 5 + [c_float] + [c_int] * 3 + [c_void_p, c_size_t, c_void_p]),
    "pa_append_kv_int8": (c_int, [c_void_p] * 6 + [c_int] * 5 + [c_void_p]),
    "pa_copy_blocks_int8": (c_int, [c_void_p] * 4 + [c_int] * 6 + [c_int64, c_int64, c_void_p]),
    "pa_append_step_int8": (c_int, [c_void_p] * 8 + [c_int] * 6 + [c_void_p]),
    "pa_swap_blocks_int8": (c_int, [c_void_p] * 7 + [c_int] * 6 + [c_int64] * 4 + [c_void_p]),
    "pa_bm_create": (c_void_p, [c_int, c_int, _P32]),
    "pa_bm_destroy": (None, [c_void_p]),
    "pa_bm_add_seq": (c_int, [c_void_p, c_int64, c_int]),
    "pa_bm_fork": (c_int, [c_void_p, c_int64, c_int64]),
    "pa_bm_append_slot": (c_int, [c_void_p, c_int64, _P32, _P32, _P32]),
    "pa_bm_append_slots": (c_int, [c_void_p, _P64, c_int, _P32, _P32, POINTER(c_int)]),
    "pa_bm_free_seq": (c_int, [c_void_p, c_int64]),
    "pa_bm_build_batch": (c_int, [c_void_p, _P64, c_int, c_int, _P32, _P32]),
    "pa_bm_shared_groups": (c_int, [c_void_p, _P64, c_int, c_int, _P32, c_int, POINTER(c_int)]),
    "pa_bm_enable_prefix_cache": (c_int, [c_void_p]),
    "pa_bm_add_seq_tokens": (c_int, [c_void_p, c_int64, _P32, c_int, POINTER(c_int)]),
    "pa_bm_append_tokens": (c_int, [c_void_p, _P64, _P32, c_int, _P32, _P32, POINTER(c_int)]),
    "pa_bm_cache_stats": (c_int, [c_void_p, POINTER(BMCacheStats)]),
    "pa_bm_idle_list": (c_int, [c_void_p, _P32, c_int, POINTER(c_int)]),
    "pa_bm_enable_host_pool": (c_int, [c_void_p, c_int, _P32]),
    "pa_bm_swap_out": (c_int, [c_void_p, _P64, c_int, _P32, c_int, POINTER(c_int)]),
    "pa_bm_swap_in": (c_int, [c_void_p, _P64, c_int, _P32, c_int, POINTER(c_int)]),
    "pa_bm_swap_stats": (c_int, [c_void_p, _P64, _P64, _P64]),
    "pa_bm_refcount": (c_int, [c_void_p, c_int]),
    "pa_bm_num_free": (c_int, [c_void_p]),
    "pa_bm_seq_len": (c_int64, [c_void_p, c_int64]),
    "pa_bm_block_table": (c_int, [c_void_p, c_int64, _P32, c_int, POINTER(c_int)]),
    "pa_bm_free_list": (c_int, [c_void_p, _P32, c_int, POINTER(c_int)]),
    "pa_bm_can_allocate": (c_int, [c_void_p, c_int]),
    "pa_bm_stats": (c_int, [c_void_p, POINTER(BMStats)]),
}
for _name, (_res, _args) in _SIGS.items():
    if HOST_ONLY and not (_name.startswith("pa_bm_") or _name in ("pa_status_string", "pa_version")):
        continue
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def _check(status: int, where: str) -> None:
    if status != PA_OK:
        raise PAError(status, where)


# ---------------------------------------------------------------------------
# device entry points (torch tensors in, data pointers across the ABI)
# ---------------------------------------------------------------------------

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise TypeError(f"unsupported element type {t.dtype}")


def _stream_ptr(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return c_void_p(stream.cuda_stream)


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return c_void_p(t.data_ptr())


def pool_shapes(num_blocks: int, hkv: int, d_head: int, block_size: int, elem_bytes: int = 2):
    """Shapes of one layer's K and V pools: [num_blocks][Hkv][B][D] each (see include/pa.h)."""
    shape = (num_blocks, hkv, block_size, d_head)
    return shape, shape


def _pool_dims(k_pool, v_pool):
    if k_pool.dim() != 4 or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("k_pool and v_pool must both be [num_blocks][Hkv][B][D]")
    nb, hkv, bs, d = k_pool.shape
    return nb, hkv, d, bs


def pa_decode_workspace_bytes(num_seqs, Hq, Hkv, d_head, block_size, max_context_len, dtype) -> int:
    return int(lib.pa_decode_workspace_bytes(num_seqs, Hq, Hkv, d_head, block_size, max_context_len, dtype))


def pa_decode_partition_tokens(num_seqs, Hq, Hkv, d_head, block_size, max_context_len, dtype) -> int:
    return int(lib.pa_decode_partition_tokens(num_seqs, Hq, Hkv, d_head, block_size, max_context_len, dtype))


def pa_decode_args(out, q, k_pool, v_pool, block_tables, context_lens, scale, max_context_len,
                   workspace=None, stream=None):
    """Validate once and return (args, workspace) for repeated ``lib.pa_decode(*args)`` calls.

    The tuple holds raw pointers: the tensors (and the returned workspace)
    must stay alive and in place while it is used.
    """
    import torch
    n, hq, d = q.shape
    nb, hkv, d2, bs = _pool_dims(k_pool, v_pool)
    if d2 != d or tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype or k_pool.dtype != q.dtype:
        raise ValueError("q, out and the pools disagree in shape or dtype")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != n or tuple(context_lens.shape) != (n,):
        raise ValueError("block_tables must be [N][max_blocks] and context_lens [N]")
    dt = _dtype_code(q)
    need = pa_decode_workspace_bytes(n, hq, hkv, d, bs, max_context_len, dt)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)  # every word is written before it is read
    ws_ptr = c_void_p(workspace.data_ptr()) if workspace is not None else c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (_dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
            _dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"),
            n, hq, hkv, d, bs, float(scale), block_tables.shape[1], int(max_context_len), nb, dt,
            ws_ptr, ws_bytes, _stream_ptr(stream))
    return args, workspace


def pa_decode(out, q, k_pool, v_pool, block_tables, context_lens, scale, max_context_len,
              workspace=None, stream=None):
    """pa_decode of include/pa.h on torch device tensors.

    q, out [N][Hq][D]; k_pool/v_pool one layer in the library layout; block_tables
    int32 [N][max_blocks]; context_lens int32 [N].  ``workspace`` is a uint8
    device tensor of at least pa_decode_workspace_bytes(...) bytes (contents need
    no initialisation); when None one is allocated through torch for this call.
    """
    args, _ws = pa_decode_args(out, q, k_pool, v_pool, block_tables, context_lens, scale, max_context_len,
                               workspace, stream)
    _check(lib.pa_decode(*args), "pa_decode")
    return out


def pa_decode_partitioned_workspace_bytes(num_seqs, Hq, Hkv, d_head, block_size, max_context_len, dtype,
                                          partition_tokens=0) -> int:
    return int(lib.pa_decode_partitioned_workspace_bytes(num_seqs, Hq, Hkv, d_head, block_size, max_context_len,
                                                         dtype, partition_tokens))


def pa_decode_partitioned(out, q, k_pool, v_pool, block_tables, context_lens, scale, max_context_len,
                          partition_tokens=0, workspace=None, stream=None):
    """pa_decode_partitioned of include/pa.h: pa_decode on the partitioned kernels (``partition_tokens`` 0 = auto)."""
    import torch
    args, _ = pa_decode_args(out, q, k_pool, v_pool, block_tables, context_lens, scale, max_context_len,
                             torch.empty(0, dtype=torch.uint8, device=q.device), stream)
    n, hq, d = q.shape
    nb, hkv, _, bs = _pool_dims(k_pool, v_pool)
    need = pa_decode_partitioned_workspace_bytes(n, hq, hkv, d, bs, max_context_len, _dtype_code(q),
                                                 partition_tokens)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)  # every word is written before it is read
    ws_ptr = c_void_p(workspace.data_ptr()) if workspace is not None else c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pa_decode_partitioned(*args[:16], int(partition_tokens), ws_ptr, ws_bytes, args[18]),
           "pa_decode_partitioned")
    return out


def pa_check_batch(block_tables, context_lens, max_context_len, num_blocks, block_size, status=None, stream=None):
    """pa_check_batch of include/pa.h: validate lengths and table entries on the device.

    Returns the int32 device tensor ``status`` of 4 words (allocated when None):
    bad rows, bad entries, first bad row, first row with a bad entry (-1 when
    none).  Read it after the stream has reached the call.
    """
    import torch
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    n = context_lens.shape[0]
    if context_lens.dim() != 1 or block_tables.dim() != 2 or block_tables.shape[0] != n:
        raise ValueError("block_tables must be [N][max_blocks] and context_lens [N]")
    if status is None:
        status = torch.empty(4, dtype=torch.int32, device=context_lens.device)
    if status.dtype != torch.int32 or status.numel() < 4:
        raise ValueError("status must hold 4 int32 words")
    _check(lib.pa_check_batch(_dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"), n,
                              block_tables.shape[1], int(max_context_len), int(num_blocks), int(block_size),
                              _dev(status, "status"), _stream_ptr(stream)), "pa_check_batch")
    return status


def pa_check_pairs(src_dst_pairs, num_blocks, status=None, stream=None):
    """pa_check_pairs of include/pa.h: validate copy-on-write pairs on the device.

    Returns the int32 device tensor ``status`` of 4 words (allocated when None):
    out-of-pool pairs, repeated destinations, destinations that are sources,
    lowest offending pair (-1 when none).
    """
    import torch
    if src_dst_pairs.dtype != torch.int32 or src_dst_pairs.dim() != 2 or src_dst_pairs.shape[1] != 2:
        raise ValueError("src_dst_pairs must be int32 [P][2]")
    if status is None:
        status = torch.empty(4, dtype=torch.int32, device=src_dst_pairs.device)
    if status.dtype != torch.int32 or status.numel() < 4:
        raise ValueError("status must hold 4 int32 words")
    p = src_dst_pairs.shape[0]
    _check(lib.pa_check_pairs(_dev(src_dst_pairs, "src_dst_pairs") if p else c_void_p(0), p, int(num_blocks),
                              _dev(status, "status"), _stream_ptr(stream)), "pa_check_pairs")
    return status


def pa_decode_step_args(out, q, k_new, v_new, k_pool, v_pool, slot_mapping, block_tables, context_lens, scale,
                        max_context_len, workspace=None, stream=None, slot_pointer=None, allocate=True):
    """Validate once and return (args, workspace) for repeated ``lib.pa_decode_step(*args)`` calls.

    ``slot_pointer`` (an int) replaces slot_mapping's data pointer, e.g. with the
    device mapping of a pinned host buffer of the same shape.
    """
    import torch
    n, hq, d = q.shape
    nb, hkv, d2, bs = _pool_dims(k_pool, v_pool)
    if d2 != d or tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype or k_pool.dtype != q.dtype:
        raise ValueError("q, out and the pools disagree in shape or dtype")
    if tuple(k_new.shape) != (n, hkv, d) or tuple(v_new.shape) != (n, hkv, d):
        raise ValueError("k_new / v_new must be [N][Hkv][D]")
    if k_new.dtype != q.dtype or v_new.dtype != q.dtype:
        raise ValueError("k_new / v_new must have q's element type")
    for t, name in ((slot_mapping, "slot_mapping"), (block_tables, "block_tables"), (context_lens, "context_lens")):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    if tuple(slot_mapping.shape) != (n,) or tuple(context_lens.shape) != (n,):
        raise ValueError("slot_mapping and context_lens must be [N]")
    if block_tables.dim() != 2 or block_tables.shape[0] != n:
        raise ValueError("block_tables must be [N][max_blocks]")
    dt = _dtype_code(q)
    need = pa_decode_workspace_bytes(n, hq, hkv, d, bs, max_context_len, dt)
    if workspace is None and need > 0 and allocate:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)  # every word is written before it is read
    ws_ptr = c_void_p(workspace.data_ptr()) if workspace is not None else c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    slots = c_void_p(slot_pointer) if slot_pointer is not None else _dev(slot_mapping, "slot_mapping")
    args = (_dev(out, "out"), _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(k_pool, "k_pool"),
            _dev(v_pool, "v_pool"), slots, _dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"),
            n, hq, hkv, d, bs, float(scale), block_tables.shape[1], int(max_context_len), nb, dt, ws_ptr, ws_bytes,
            _stream_ptr(stream))
    return args, workspace


def pa_decode_step(out, q, k_new, v_new, k_pool, v_pool, slot_mapping, block_tables, context_lens, scale,
                   max_context_len, workspace=None, stream=None):
    """pa_decode_step of include/pa.h: store each row's new token, advance the rows, and decode with it."""
    args, _ws = pa_decode_step_args(out, q, k_new, v_new, k_pool, v_pool, slot_mapping, block_tables, context_lens,
                                    scale, max_context_len, workspace, stream)
    _check(lib.pa_decode_step(*args), "pa_decode_step")
    return out


PA_NOALLOC_SCRATCH_BYTES = 8 << 20  # the fixed device array of pa_decode_step_noalloc (include/pa.h)


def pa_decode_step_noalloc(out, q, k_new, v_new, k_pool, v_pool, slot_mapping, block_tables, context_lens, scale,
                           max_context_len, stream=None):
    """pa_decode_step_noalloc of include/pa.h: pa_decode_step with the library's fixed device workspace.

    Allocates nothing, here or in the library: the argument checks are those of
    pa_decode_step_args without its workspace.
    """
    args, _ = pa_decode_step_args(out, q, k_new, v_new, k_pool, v_pool, slot_mapping, block_tables, context_lens,
                                  scale, max_context_len, stream=stream, allocate=False)
    _check(lib.pa_decode_step_noalloc(*args[:19], args[21]), "pa_decode_step_noalloc")
    return out


def pa_decode_shared_workspace_bytes(num_seqs, num_groups, Hq, Hkv, d_head, block_size, max_context_len,
                                     dtype) -> int:
    return int(lib.pa_decode_shared_workspace_bytes(num_seqs, num_groups, Hq, Hkv, d_head, block_size,
                                                    max_context_len, dtype))


def _groups_arg(groups, groups_pointer):
    """(pointer, count) of an int32 [G][3] device tensor of groups, or of a mapped host buffer."""
    import torch
    if groups is None:
        return c_void_p(0), 0
    if groups.dtype != torch.int32 or groups.dim() != 2 or groups.shape[1] != 3:
        raise ValueError("groups must be int32 [G][3] (first row, rows, shared tokens)")
    g = groups.shape[0]
    if groups_pointer is not None:
        return c_void_p(groups_pointer), g
    return (_dev(groups, "groups") if g else c_void_p(0)), g


def pa_decode_shared_args(out, q, k_pool, v_pool, block_tables, context_lens, groups, scale, max_context_len,
                          workspace=None, stream=None, groups_pointer=None):
    """Validate once and return (args, workspace) for repeated ``lib.pa_decode_shared(*args)`` calls.

    ``groups`` is int32 [G][3] (device, or ``groups_pointer`` = the device
    mapping of a pinned host buffer of that shape).
    """
    import torch
    base, _ = pa_decode_args(out, q, k_pool, v_pool, block_tables, context_lens, scale, max_context_len,
                             torch.empty(0, dtype=torch.uint8, device=q.device), stream)
    gp, ng = _groups_arg(groups, groups_pointer)
    n, hq, d = q.shape
    nb, hkv, _, bs = _pool_dims(k_pool, v_pool)
    need = pa_decode_shared_workspace_bytes(n, ng, hq, hkv, d, bs, max_context_len, _dtype_code(q))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)  # every word is written before it is read
    ws_ptr = c_void_p(workspace.data_ptr()) if workspace is not None else c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = base[:6] + (gp, ng) + base[6:16] + (ws_ptr, ws_bytes, base[18])
    return args, workspace


def pa_decode_shared(out, q, k_pool, v_pool, block_tables, context_lens, groups, scale, max_context_len,
                     workspace=None, stream=None):
    """pa_decode_shared of include/pa.h: pa_decode with each group's shared full blocks read once."""
    args, _ws = pa_decode_shared_args(out, q, k_pool, v_pool, block_tables, context_lens, groups, scale,
                                      max_context_len, workspace, stream)
    _check(lib.pa_decode_shared(*args), "pa_decode_shared")
    return out


def pa_decode_step_shared_args(out, q, k_new, v_new, k_pool, v_pool, slot_mapping, block_tables, context_lens,
                               groups, scale, max_context_len, workspace=None, stream=None, slot_pointer=None,
                               groups_pointer=None):
    """Validate once and return (args, workspace) for repeated ``lib.pa_decode_step_shared(*args)`` calls."""
    import torch
    base, _ = pa_decode_step_args(out, q, k_new, v_new, k_pool, v_pool, slot_mapping, block_tables, context_lens,
                                  scale, max_context_len, torch.empty(0, dtype=torch.uint8, device=q.device),
                                  stream, slot_pointer)
    gp, ng = _groups_arg(groups, groups_pointer)
    n, hq, d = q.shape
    nb, hkv, _, bs = _pool_dims(k_pool, v_pool)
    need = pa_decode_shared_workspace_bytes(n, ng, hq, hkv, d, bs, max_context_len, _dtype_code(q))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)  # every word is written before it is read
    ws_ptr = c_void_p(workspace.data_ptr()) if workspace is not None else c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = base[:9] + (gp, ng) + base[9:19] + (ws_ptr, ws_bytes, base[21])
    return args, workspace


def pa_decode_step_shared(out, q, k_new, v_new, k_pool, v_pool, slot_mapping, block_tables, context_lens, groups,
                          scale, max_context_len, workspace=None, stream=None):
    """pa_decode_step_shared of include/pa.h: pa_decode_step with each group's shared full blocks read once."""
    args, _ws = pa_decode_step_shared_args(out, q, k_new, v_new, k_pool, v_pool, slot_mapping, block_tables,
                                           context_lens, groups, scale, max_context_len, workspace, stream)
    _check(lib.pa_decode_step_shared(*args), "pa_decode_step_shared")
    return out


def pa_append_kv_args(k_pool, v_pool, k_new, v_new, slot_mapping, stream=None):
    """Validate once and return the argument tuple for repeated ``lib.pa_append_kv(*args)`` calls."""
    import torch
    nb, hkv, d, bs = _pool_dims(k_pool, v_pool)
    t = k_new.shape[0]
    if tuple(k_new.shape) != (t, hkv, d) or tuple(v_new.shape) != (t, hkv, d):
        raise ValueError("k_new / v_new must be [T][Hkv][D]")
    if k_new.dtype != k_pool.dtype or v_new.dtype != k_pool.dtype:
        raise ValueError("k_new / v_new must have the pool's element type")
    if slot_mapping.dtype != torch.int32 or tuple(slot_mapping.shape) != (t,):
        raise ValueError("slot_mapping must be int32 [T]")
    return (_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
            _dev(slot_mapping, "slot_mapping"), t, hkv, d, bs, nb, _dtype_code(k_pool), _stream_ptr(stream))


def pa_append_kv(k_pool, v_pool, k_new, v_new, slot_mapping, stream=None):
    """pa_append_kv of include/pa.h: k_new/v_new [T][Hkv][D], slot_mapping int32 [T]."""
    _check(lib.pa_append_kv(*pa_append_kv_args(k_pool, v_pool, k_new, v_new, slot_mapping, stream)),
           "pa_append_kv")


def pa_append_step_args(k_pool, v_pool, k_new, v_new, slot_mapping, block_tables, context_lens, stream=None):
    """Validate once and return the argument tuple for repeated ``lib.pa_append_step(*args)`` calls."""
    import torch
    nb, hkv, d, bs = _pool_dims(k_pool, v_pool)
    n = k_new.shape[0]
    if tuple(k_new.shape) != (n, hkv, d) or tuple(v_new.shape) != (n, hkv, d):
        raise ValueError("k_new / v_new must be [N][Hkv][D]")
    if k_new.dtype != k_pool.dtype or v_new.dtype != k_pool.dtype:
        raise ValueError("k_new / v_new must have the pool's element type")
    for t, name in ((slot_mapping, "slot_mapping"), (block_tables, "block_tables"), (context_lens, "context_lens")):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    if tuple(slot_mapping.shape) != (n,) or tuple(context_lens.shape) != (n,):
        raise ValueError("slot_mapping and context_lens must be [N]")
    if block_tables.dim() != 2 or block_tables.shape[0] != n:
        raise ValueError("block_tables must be [N][max_blocks]")
    return (_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
            _dev(slot_mapping, "slot_mapping"), _dev(block_tables, "block_tables"),
            _dev(context_lens, "context_lens"), n, block_tables.shape[1], hkv, d, bs, nb, _dtype_code(k_pool),
            _stream_ptr(stream))


def pa_append_step(k_pool, v_pool, k_new, v_new, slot_mapping, block_tables, context_lens, stream=None):
    """pa_append_step of include/pa.h: append row n's token at slot_mapping[n] and advance
    block_tables[n] / context_lens[n] (device tensors, updated in place)."""
    _check(lib.pa_append_step(*pa_append_step_args(k_pool, v_pool, k_new, v_new, slot_mapping, block_tables,
                                                   context_lens, stream)), "pa_append_step")


def pa_copy_blocks_args(k_pool, v_pool, src_dst_pairs, stream=None):
    """Validate once and return the argument tuple for ``lib.pa_copy_blocks(*args)``.

    Pools are one layer ([num_blocks]...) or all layers ([L][num_blocks]...);
    src_dst_pairs is an int32 device tensor [P][2] (P may be lowered in the
    returned tuple's 4th entry to use a prefix of the pairs).
    """
    import torch
    layered = k_pool.dim() == 5
    kl, vl = (k_pool[0], v_pool[0]) if layered else (k_pool, v_pool)
    nb, hkv, d, bs = _pool_dims(kl, vl)
    layers = k_pool.shape[0] if layered else 1
    if src_dst_pairs.dtype != torch.int32 or src_dst_pairs.dim() != 2 or src_dst_pairs.shape[1] != 2:
        raise ValueError("src_dst_pairs must be int32 [P][2]")
    stride = kl.numel() if layered else 0
    return (_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), _dev(src_dst_pairs, "src_dst_pairs"),
            src_dst_pairs.shape[0], hkv, d, bs, nb, layers, stride, _dtype_code(k_pool), _stream_ptr(stream))


def pa_copy_blocks(k_pool, v_pool, src_dst_pairs, stream=None):
    """pa_copy_blocks of include/pa.h."""
    _check(lib.pa_copy_blocks(*pa_copy_blocks_args(k_pool, v_pool, src_dst_pairs, stream)), "pa_copy_blocks")


# ---------------------------------------------------------------------------
# swapping: blocks between the device pool and a pinned host pool
# ---------------------------------------------------------------------------

_HIP = None


def host_device_pointer(t) -> int:
    """Device address of a pinned host tensor's memory (hipHostGetDevicePointer), for kernels that read or write
    it over PCIe."""
    global _HIP
    if not t.is_pinned():
        raise ValueError("host pools must be pinned (torch.empty(..., pin_memory=True))")
    if _HIP is None:
        _HIP = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch has loaded
    dp = c_void_p()
    if _HIP.hipHostGetDevicePointer(ctypes.byref(dp), c_void_p(t.data_ptr()), 0) != 0 or not dp.value:
        raise PAError(PA_ERR_HIP, "hipHostGetDevicePointer")
    return dp.value


def _pool_ptr(t, name):
    """Device pointer of a pool: a device tensor's data, or the mapping of a pinned host tensor."""
    if t.is_cuda:
        return _dev(t, name)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return c_void_p(host_device_pointer(t))


def _layers(k_pool):
    """(layers, blocks per layer, elements per layer) of a one-layer [nb]... or layered [L][nb]... K pool."""
    if k_pool.dim() == 5:
        return k_pool.shape[0], k_pool.shape[1], k_pool[0].numel()
    return 1, k_pool.shape[0], k_pool.numel()


def pa_swap_blocks(dst_k, dst_v, src_k, src_v, pairs, stream=None):
    """pa_swap_blocks of include/pa.h.  Pools: device tensors or pinned host tensors of the library layout,
    one layer [nb]... or layered [L][nb]...; pairs: int32 [P][2] device tensor (src block, dst block)."""
    import torch
    if pairs.dtype != torch.int32 or pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be int32 [P][2]")
    ls, nbs, es = _layers(src_k)
    ld, nbd, ed = _layers(dst_k)
    if ls != ld or src_k.dtype != dst_k.dtype:
        raise ValueError("pools disagree in layers or element type")
    kl = src_k[0] if src_k.dim() == 5 else src_k
    vl = src_v[0] if src_v.dim() == 5 else src_v
    _, hkv, d, bs = _pool_dims(kl, vl)
    _check(lib.pa_swap_blocks(_pool_ptr(dst_k, "dst_k"), _pool_ptr(dst_v, "dst_v"), _pool_ptr(src_k, "src_k"),
                              _pool_ptr(src_v, "src_v"), _dev(pairs, "pairs") if pairs.shape[0] else c_void_p(0),
                              pairs.shape[0], hkv, d, bs, _dtype_code(src_k), nbs, nbd, ls, es, ed,
                              _stream_ptr(stream)), "pa_swap_blocks")


def _swap_codes(fn, name, dst_k, dst_v, dst_scales, src_k, src_v, src_scales, pairs, stream):
    import torch
    if pairs.dtype != torch.int32 or pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be int32 [P][2]")
    nbs, hkv, d, bs = _fp8_pools(src_k, src_v)
    nbd, _, _, _ = _fp8_pools(dst_k, dst_v)
    _scales(src_scales, nbs, hkv)
    _scales(dst_scales, nbd, hkv)
    _check(fn(_pool_ptr(dst_k, "dst_k"), _pool_ptr(dst_v, "dst_v"), _pool_ptr(dst_scales, "dst_scales"),
              _pool_ptr(src_k, "src_k"), _pool_ptr(src_v, "src_v"), _pool_ptr(src_scales, "src_scales"),
              _dev(pairs, "pairs") if pairs.shape[0] else c_void_p(0), pairs.shape[0], hkv, d, bs,
              nbs, nbd, 1, 0, 0, 0, 0, _stream_ptr(stream)), name)


def pa_swap_blocks_fp8(dst_k, dst_v, dst_scales, src_k, src_v, src_scales, pairs, stream=None):
    """pa_swap_blocks_fp8 of include/pa.h (one-layer FP8 pools with their [nb][Hkv][2] scales)."""
    _swap_codes(lib.pa_swap_blocks_fp8, "pa_swap_blocks_fp8", dst_k, dst_v, dst_scales, src_k, src_v, src_scales,
                pairs, stream)


def pa_swap_blocks_int8(dst_k, dst_v, dst_scales, src_k, src_v, src_scales, pairs, stream=None):
    """pa_swap_blocks_int8 of include/pa.h (one-layer INT8 pools with their [nb][Hkv][2] scales)."""
    _swap_codes(lib.pa_swap_blocks_int8, "pa_swap_blocks_int8", dst_k, dst_v, dst_scales, src_k, src_v, src_scales,
                pairs, stream)


# ---------------------------------------------------------------------------
# FP8 (E4M3) and INT8 caches: uint8 code pools [num_blocks][Hkv][B][D]
# and one float32 scale array [num_blocks][Hkv][2] (key, value; or
# [L][num_blocks][Hkv][2] for a layered copy); the INT8 functions take the same
# arguments as the FP8 ones
# ---------------------------------------------------------------------------

def _fp8_pools(k_pool, v_pool):
    import torch
    if k_pool.dtype != torch.uint8 or v_pool.dtype != torch.uint8:
        raise ValueError("code pools hold uint8 bytes")
    return _pool_dims(k_pool, v_pool)


def _scales(scales, nb, hkv, lead=()):
    import torch
    want = tuple(lead) + (nb, hkv, 2)
    if scales.dtype != torch.float32 or tuple(scales.shape) != want or not scales.is_contiguous():
        raise ValueError(f"scales must be contiguous float32 {list(want)} (key, value)")


def pa_decode_fp8_args(out, q, k_pool, v_pool, scales, block_tables, context_lens, scale,
                       max_context_len, workspace=None, stream=None):
    """Validate once and return (args, workspace) for repeated ``lib.pa_decode_fp8(*args)`` calls."""
    return _decode_codes_args(PA_FP8_E4M3, out, q, k_pool, v_pool, scales, block_tables, context_lens,
                              scale, max_context_len, workspace, stream)


def pa_decode_int8_args(out, q, k_pool, v_pool, scales, block_tables, context_lens, scale,
                        max_context_len, workspace=None, stream=None):
    """Validate once and return (args, workspace) for repeated ``lib.pa_decode_int8(*args)`` calls."""
    return _decode_codes_args(PA_INT8, out, q, k_pool, v_pool, scales, block_tables, context_lens,
                              scale, max_context_len, workspace, stream)


def _decode_codes_args(dtype_code, out, q, k_pool, v_pool, scales, block_tables, context_lens, scale,
                       max_context_len, workspace, stream):
    import torch
    n, hq, d = q.shape
    nb, hkv, d2, bs = _fp8_pools(k_pool, v_pool)
    _scales(scales, nb, hkv)
    if q.dtype != torch.bfloat16 or out.dtype != torch.bfloat16 or tuple(out.shape) != tuple(q.shape) or d2 != d:
        raise ValueError("q and out must be bf16 [N][Hq][D] matching the pools")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != n or tuple(context_lens.shape) != (n,):
        raise ValueError("block_tables must be [N][max_blocks] and context_lens [N]")
    need = pa_decode_workspace_bytes(n, hq, hkv, d, bs, max_context_len, dtype_code)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)  # every word is written before it is read
    ws_ptr = c_void_p(workspace.data_ptr()) if workspace is not None else c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (_dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
            _dev(scales, "scales"), _dev(block_tables, "block_tables"),
            _dev(context_lens, "context_lens"), n, hq, hkv, d, bs, float(scale), block_tables.shape[1],
            int(max_context_len), nb, ws_ptr, ws_bytes, _stream_ptr(stream))
    return args, workspace


def pa_decode_fp8(out, q, k_pool, v_pool, scales, block_tables, context_lens, scale, max_context_len,
                  workspace=None, stream=None):
    """pa_decode_fp8 of include/pa.h: bf16 q/out over uint8 E4M3 code pools with float32 scales."""
    args, _ws = pa_decode_fp8_args(out, q, k_pool, v_pool, scales, block_tables, context_lens, scale,
                                   max_context_len, workspace, stream)
    _check(lib.pa_decode_fp8(*args), "pa_decode_fp8")
    return out


def pa_decode_int8(out, q, k_pool, v_pool, scales, block_tables, context_lens, scale, max_context_len,
                   workspace=None, stream=None):
    """pa_decode_int8 of include/pa.h: bf16 q/out over INT8 code pools (uint8 bytes) with float32 scales."""
    args, _ws = pa_decode_int8_args(out, q, k_pool, v_pool, scales, block_tables, context_lens, scale,
                                    max_context_len, workspace, stream)
    _check(lib.pa_decode_int8(*args), "pa_decode_int8")
    return out


def _decode_step_codes_args(dtype_code, out, q, k_new, v_new, k_pool, v_pool, scales, slot_mapping,
                            block_tables, context_lens, scale, max_context_len, workspace, stream, slot_pointer):
    import torch
    args, workspace = _decode_codes_args(dtype_code, out, q, k_pool, v_pool, scales, block_tables,
                                         context_lens, scale, max_context_len, workspace, stream)
    n, hq, d = q.shape
    hkv = scales.shape[1]
    if tuple(k_new.shape) != (n, hkv, d) or tuple(v_new.shape) != (n, hkv, d):
        raise ValueError("k_new / v_new must be [N][Hkv][D]")
    if k_new.dtype != torch.bfloat16 or v_new.dtype != torch.bfloat16:
        raise ValueError("k_new / v_new must be bf16")
    if slot_mapping.dtype != torch.int32 or tuple(slot_mapping.shape) != (n,):
        raise ValueError("slot_mapping must be int32 [N]")
    slots = c_void_p(slot_pointer) if slot_pointer is not None else _dev(slot_mapping, "slot_mapping")
    # pa_decode_*(out, q, k, v, scales, tables, lens, ...) -> pa_decode_step_*(out, q, k_new, v_new, k, v, scales,
    # slots, tables, lens, ...)
    return (args[:2] + (_dev(k_new, "k_new"), _dev(v_new, "v_new")) + args[2:5] + (slots,) + args[5:]), workspace


def pa_decode_step_fp8_args(out, q, k_new, v_new, k_pool, v_pool, scales, slot_mapping, block_tables,
                            context_lens, scale, max_context_len, workspace=None, stream=None, slot_pointer=None):
    """Validate once and return (args, workspace) for repeated ``lib.pa_decode_step_fp8(*args)`` calls."""
    return _decode_step_codes_args(PA_FP8_E4M3, out, q, k_new, v_new, k_pool, v_pool, scales,
                                   slot_mapping, block_tables, context_lens, scale, max_context_len, workspace,
                                   stream, slot_pointer)


def pa_decode_step_int8_args(out, q, k_new, v_new, k_pool, v_pool, scales, slot_mapping, block_tables,
                             context_lens, scale, max_context_len, workspace=None, stream=None, slot_pointer=None):
    """Validate once and return (args, workspace) for repeated ``lib.pa_decode_step_int8(*args)`` calls."""
    return _decode_step_codes_args(PA_INT8, out, q, k_new, v_new, k_pool, v_pool, scales, slot_mapping,
                                   block_tables, context_lens, scale, max_context_len, workspace, stream,
                                   slot_pointer)


def pa_decode_step_fp8(out, q, k_new, v_new, k_pool, v_pool, scales, slot_mapping, block_tables,
                       context_lens, scale, max_context_len, workspace=None, stream=None):
    """pa_decode_step_fp8 of include/pa.h: attend to each row's new token as its codes, then store them."""
    args, _ws = pa_decode_step_fp8_args(out, q, k_new, v_new, k_pool, v_pool, scales, slot_mapping,
                                        block_tables, context_lens, scale, max_context_len, workspace, stream)
    _check(lib.pa_decode_step_fp8(*args), "pa_decode_step_fp8")
    return out


def pa_decode_step_int8(out, q, k_new, v_new, k_pool, v_pool, scales, slot_mapping, block_tables,
                        context_lens, scale, max_context_len, workspace=None, stream=None):
    """pa_decode_step_int8 of include/pa.h: as pa_decode_step_fp8 over an INT8 cache."""
    args, _ws = pa_decode_step_int8_args(out, q, k_new, v_new, k_pool, v_pool, scales, slot_mapping,
                                         block_tables, context_lens, scale, max_context_len, workspace, stream)
    _check(lib.pa_decode_step_int8(*args), "pa_decode_step_int8")
    return out


def pa_append_kv_fp8_args(k_pool, v_pool, scales, k_new, v_new, slot_mapping, stream=None):
    """Validate once and return the argument tuple for ``lib.pa_append_kv_fp8(*args)``."""
    import torch
    nb, hkv, d, bs = _fp8_pools(k_pool, v_pool)
    _scales(scales, nb, hkv)
    t = k_new.shape[0]
    if tuple(k_new.shape) != (t, hkv, d) or tuple(v_new.shape) != (t, hkv, d):
        raise ValueError("k_new / v_new must be [T][Hkv][D]")
    if k_new.dtype != torch.bfloat16 or v_new.dtype != torch.bfloat16:
        raise ValueError("k_new / v_new must be bf16")
    if slot_mapping.dtype != torch.int32 or tuple(slot_mapping.shape) != (t,):
        raise ValueError("slot_mapping must be int32 [T]")
    return (_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), _dev(scales, "scales"),
            _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(slot_mapping, "slot_mapping"), t, hkv, d, bs, nb,
            _stream_ptr(stream))


def pa_append_kv_fp8(k_pool, v_pool, scales, k_new, v_new, slot_mapping, stream=None):
    """pa_append_kv_fp8 of include/pa.h: quantize bf16 k_new/v_new [T][Hkv][D] into their slots."""
    _check(lib.pa_append_kv_fp8(*pa_append_kv_fp8_args(k_pool, v_pool, scales, k_new, v_new,
                                                       slot_mapping, stream)), "pa_append_kv_fp8")


def pa_append_kv_int8(k_pool, v_pool, scales, k_new, v_new, slot_mapping, stream=None):
    """pa_append_kv_int8 of include/pa.h: quantize bf16 k_new/v_new [T][Hkv][D] into their slots as INT8 codes."""
    _check(lib.pa_append_kv_int8(*pa_append_kv_fp8_args(k_pool, v_pool, scales, k_new, v_new,
                                                        slot_mapping, stream)), "pa_append_kv_int8")


def pa_append_step_fp8_args(k_pool, v_pool, scales, k_new, v_new, slot_mapping, block_tables,
                            context_lens, stream=None):
    """Validate once and return the argument tuple for ``lib.pa_append_step_fp8(*args)``."""
    import torch
    nb, hkv, d, bs = _fp8_pools(k_pool, v_pool)
    _scales(scales, nb, hkv)
    n = k_new.shape[0]
    if tuple(k_new.shape) != (n, hkv, d) or tuple(v_new.shape) != (n, hkv, d):
        raise ValueError("k_new / v_new must be [N][Hkv][D]")
    if k_new.dtype != torch.bfloat16 or v_new.dtype != torch.bfloat16:
        raise ValueError("k_new / v_new must be bf16")
    for t, name in ((slot_mapping, "slot_mapping"), (block_tables, "block_tables"), (context_lens, "context_lens")):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    if tuple(slot_mapping.shape) != (n,) or tuple(context_lens.shape) != (n,):
        raise ValueError("slot_mapping and context_lens must be [N]")
    if block_tables.dim() != 2 or block_tables.shape[0] != n:
        raise ValueError("block_tables must be [N][max_blocks]")
    return (_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), _dev(scales, "scales"),
            _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(slot_mapping, "slot_mapping"),
            _dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"), n, block_tables.shape[1], hkv, d,
            bs, nb, _stream_ptr(stream))


def pa_append_step_fp8(k_pool, v_pool, scales, k_new, v_new, slot_mapping, block_tables, context_lens,
                       stream=None):
    """pa_append_step_fp8 of include/pa.h: quantizing append of row n's token and the row moved forward."""
    _check(lib.pa_append_step_fp8(*pa_append_step_fp8_args(k_pool, v_pool, scales, k_new, v_new,
                                                           slot_mapping, block_tables, context_lens, stream)),
           "pa_append_step_fp8")


def pa_append_step_int8(k_pool, v_pool, scales, k_new, v_new, slot_mapping, block_tables, context_lens,
                        stream=None):
    """pa_append_step_int8 of include/pa.h: INT8 quantizing append of row n's token and the row moved forward."""
    _check(lib.pa_append_step_int8(*pa_append_step_fp8_args(k_pool, v_pool, scales, k_new, v_new,
                                                            slot_mapping, block_tables, context_lens, stream)),
           "pa_append_step_int8")


def pa_copy_blocks_fp8_args(k_pool, v_pool, scales, src_dst_pairs, stream=None):
    """Validate once and return the argument tuple for ``lib.pa_copy_blocks_fp8(*args)``.

    Pools and scales are one layer or all layers (leading [L] on both).
    """
    import torch
    layered = k_pool.dim() == 5
    kl, vl = (k_pool[0], v_pool[0]) if layered else (k_pool, v_pool)
    nb, hkv, d, bs = _fp8_pools(kl, vl)
    layers = k_pool.shape[0] if layered else 1
    _scales(scales, nb, hkv, (layers,) if layered else ())
    if src_dst_pairs.dtype != torch.int32 or src_dst_pairs.dim() != 2 or src_dst_pairs.shape[1] != 2:
        raise ValueError("src_dst_pairs must be int32 [P][2]")
    stride = kl.numel() if layered else 0
    sstride = nb * hkv * 2 if layered else 0
    return (_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), _dev(scales, "scales"),
            _dev(src_dst_pairs, "src_dst_pairs"), src_dst_pairs.shape[0], hkv, d, bs, nb, layers, stride, sstride,
            _stream_ptr(stream))


def pa_copy_blocks_fp8(k_pool, v_pool, scales, src_dst_pairs, stream=None):
    """pa_copy_blocks_fp8 of include/pa.h: codes and scales of each src block over its dst."""
    _check(lib.pa_copy_blocks_fp8(*pa_copy_blocks_fp8_args(k_pool, v_pool, scales, src_dst_pairs, stream)),
           "pa_copy_blocks_fp8")


def pa_copy_blocks_int8(k_pool, v_pool, scales, src_dst_pairs, stream=None):
    """pa_copy_blocks_int8 of include/pa.h: INT8 codes and scales of each src block over its dst."""
    _check(lib.pa_copy_blocks_int8(*pa_copy_blocks_fp8_args(k_pool, v_pool, scales, src_dst_pairs,
                                                            stream)), "pa_copy_blocks_int8")


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr32(a):
    return a.ctypes.data_as(_P32)


class BlockManager:
    """Owning wrapper of a pa_bm handle; each method is one pa_bm_* call."""

    def __init__(self, num_blocks: int, block_size: int, pop_order=None):
        order = None if pop_order is None else _i32(pop_order)
        if order is not None and order.shape != (num_blocks,):
            raise ValueError("pop_order must hold num_blocks entries")
        self._h = lib.pa_bm_create(num_blocks, block_size, None if order is None else _ptr32(order))
        if not self._h:
            raise PAError(PA_ERR_INVALID_ARG, "pa_bm_create")
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self):
        if self._h:
            lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_seq(self, seq: int, num_tokens: int) -> int:
        return lib.pa_bm_add_seq(self._h, seq, num_tokens)

    def fork(self, parent: int, child: int) -> int:
        return lib.pa_bm_fork(self._h, parent, child)

    def append_slot(self, seq: int):
        slot, src, dst = c_int32(), c_int32(), c_int32()
        st = lib.pa_bm_append_slot(self._h, seq, ctypes.byref(slot), ctypes.byref(src), ctypes.byref(dst))
        return st, slot.value, src.value, dst.value

    def append_slots(self, seqs):
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        n = s.shape[0]
        slots = np.empty(max(n, 1), dtype=np.int32)
        pairs = np.empty((max(n, 1), 2), dtype=np.int32)
        npairs = c_int()
        st = lib.pa_bm_append_slots(self._h, s.ctypes.data_as(_P64), n, _ptr32(slots), _ptr32(pairs),
                                    ctypes.byref(npairs))
        if st != PA_OK:
            return st, slots[:0], pairs[:0], -npairs.value - 1
        return st, slots[:n], pairs[:npairs.value], -1

    def enable_prefix_cache(self) -> int:
        return lib.pa_bm_enable_prefix_cache(self._h)

    def add_seq_tokens(self, seq: int, tokens):
        """(status, cached tokens reused) of pa_bm_add_seq_tokens."""
        t = _i32(tokens)
        hit = c_int()
        st = lib.pa_bm_add_seq_tokens(self._h, seq, _ptr32(t), t.shape[0], ctypes.byref(hit))
        return st, hit.value

    def append_tokens(self, seqs, tokens=None):
        """pa_bm_append_tokens: (status, slots, cow pairs, failing index or -1); tokens None = unknown ids."""
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        n = s.shape[0]
        t = None if tokens is None else _i32(tokens)
        slots = np.empty(max(n, 1), dtype=np.int32)
        pairs = np.empty((max(n, 1), 2), dtype=np.int32)
        npairs = c_int()
        st = lib.pa_bm_append_tokens(self._h, s.ctypes.data_as(_P64), None if t is None else _ptr32(t), n,
                                     _ptr32(slots), _ptr32(pairs), ctypes.byref(npairs))
        if st != PA_OK:
            return st, slots[:0], pairs[:0], -npairs.value - 1
        return st, slots[:n], pairs[:npairs.value], -1

    def cache_stats(self):
        out = BMCacheStats()
        _check(lib.pa_bm_cache_stats(self._h, ctypes.byref(out)), "pa_bm_cache_stats")
        return out.as_dict()

    def idle_list(self):
        n = c_int()
        cap = max(self.num_blocks, 1)
        out = np.empty(cap, dtype=np.int32)
        st = lib.pa_bm_idle_list(self._h, _ptr32(out), cap, ctypes.byref(n))
        return out[: n.value].tolist() if st == PA_OK else []

    def enable_host_pool(self, num_host_blocks: int, pop_order=None) -> int:
        order = None if pop_order is None else _i32(pop_order)
        return lib.pa_bm_enable_host_pool(self._h, num_host_blocks, None if order is None else _ptr32(order))

    def _swap(self, fn, seqs):
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        n = s.shape[0]
        cap = max(sum(self.block_table(int(x))[1].__len__() for x in s), 1)
        pairs = np.empty((cap, 2), dtype=np.int32)
        npairs = c_int()
        st = fn(self._h, s.ctypes.data_as(_P64), n, _ptr32(pairs), cap, ctypes.byref(npairs))
        return st, pairs[: npairs.value].copy() if st == PA_OK else np.zeros((0, 2), dtype=np.int32)

    def swap_out(self, seqs):
        """(status, int32 [P][2] (device block, host block)) of pa_bm_swap_out."""
        return self._swap(lib.pa_bm_swap_out, seqs)

    def swap_in(self, seqs):
        """(status, int32 [P][2] (host block, device block)) of pa_bm_swap_in."""
        return self._swap(lib.pa_bm_swap_in, seqs)

    def swap_stats(self):
        a, b, c = c_int64(), c_int64(), c_int64()
        _check(lib.pa_bm_swap_stats(self._h, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)), "pa_bm_swap_stats")
        return {"num_swapped": a.value, "host_free": b.value, "host_blocks": c.value}

    @property
    def handle(self):
        """The pa_bm* handle, for direct ``lib.pa_bm_*`` calls with caller-owned host buffers."""
        return self._h

    def free_seq(self, seq: int) -> int:
        return lib.pa_bm_free_seq(self._h, seq)

    def build_batch(self, seqs, max_blocks: int):
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        n = s.shape[0]
        tables = np.zeros((n, max_blocks), dtype=np.int32)
        lens = np.zeros(n, dtype=np.int32)
        st = lib.pa_bm_build_batch(self._h, s.ctypes.data_as(_P64), n, max_blocks, _ptr32(tables), _ptr32(lens))
        return st, tables, lens

    def shared_groups(self, seqs, max_members: int):
        """(status, int32 [G][3] groups (first row, rows, shared tokens)) of pa_bm_shared_groups."""
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        n = s.shape[0]
        cap = max(n // 2, 1)
        out = np.zeros((cap, 3), dtype=np.int32)
        g = c_int()
        st = lib.pa_bm_shared_groups(self._h, s.ctypes.data_as(_P64), n, max_members, _ptr32(out), cap,
                                     ctypes.byref(g))
        return st, out[: g.value].copy() if st == PA_OK else np.zeros((0, 3), dtype=np.int32)

    def refcount(self, block: int) -> int:
        return lib.pa_bm_refcount(self._h, block)

    def num_free(self) -> int:
        return lib.pa_bm_num_free(self._h)

    def seq_len(self, seq: int) -> int:
        return lib.pa_bm_seq_len(self._h, seq)

    def block_table(self, seq: int):
        n = c_int()
        cap = max(self.num_blocks, 1)
        out = np.empty(cap, dtype=np.int32)
        st = lib.pa_bm_block_table(self._h, seq, _ptr32(out), cap, ctypes.byref(n))
        return st, out[: n.value].tolist() if st == PA_OK else []

    def free_list(self):
        n = c_int()
        out = np.empty(max(self.num_blocks, 1), dtype=np.int32)
        st = lib.pa_bm_free_list(self._h, _ptr32(out), out.shape[0], ctypes.byref(n))
        _check(st, "pa_bm_free_list")
        return out[: n.value].tolist()

    def can_allocate(self, num_tokens: int) -> bool:
        return bool(lib.pa_bm_can_allocate(self._h, num_tokens))

    def stats(self):
        s = BMStats()
        _check(lib.pa_bm_stats(self._h, ctypes.byref(s)), "pa_bm_stats")
        return s.as_dict()

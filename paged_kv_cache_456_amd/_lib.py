"""ctypes binding of libpa.so: the same entry points as include/pa.h, taking torch
tensors. Only argument marshalling happens here (shapes, dtypes, data pointers,
the current HIP stream); every step of the computation runs in the library's
HIP kernels. There is no CPU fallback: without the built library, or with
tensors that are not on a GPU, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")

PA_F32, PA_BF16 = 0, 1
PA_OK, PA_EINVAL, PA_EUNSUPPORTED, PA_EWORKSPACE, PA_EHIP, PA_ENOSPACE = 0, 1, 2, 3, 4, 5

EXPORTS = ("pa_reshape_and_cache", "pa_copy_blocks", "pa_swap_blocks", "pa_decode", "pa_decode_partitioned",
           "pa_decode_partitioned_workspace_size", "pa_decode_partitioned_noalloc",
           "pa_decode_balanced", "pa_decode_balanced_workspace_size", "pa_decode_step",
           "pa_decode_partitioned_step",
           "pa_decode_cascade",
           "pa_decode_cascade_workspace_size", "pa_prefill", "pa_prefill_workspace_size",
           "pa_stream_read", "pa_status_str",
           "pa_bm_create", "pa_bm_destroy", "pa_bm_add_sequence", "pa_bm_append_token",
           "pa_bm_fork", "pa_bm_free_sequence", "pa_bm_num_free_blocks", "pa_bm_length",
           "pa_bm_block_table")

_lib: Optional[ctypes.CDLL] = None


class PagedAttentionError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_str(status)} (status {status})")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libpa.so (after torch, so that both share one HIP runtime) and declare
    the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                           "or python -m paged_kv_cache_456_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.pa_reshape_and_cache.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i32, i64, i32, vp]
    lib.pa_reshape_and_cache.restype = i32
    lib.pa_copy_blocks.argtypes = [vp, vp, vp, i64, i32, i32, i32, i64, i32, vp]
    lib.pa_copy_blocks.restype = i32
    lib.pa_swap_blocks.argtypes = [vp, vp, i64, vp, vp, i64, vp, i64, i32, i32, i32, i32, vp]
    lib.pa_swap_blocks.restype = i32
    lib.pa_stream_read.argtypes = [vp, i64, vp, i32, vp]
    lib.pa_stream_read.restype = i32
    lib.pa_decode.argtypes = [vp, i32, vp, vp, vp, i32, vp, i32, vp, i32, i32, i32, i32, i32, i64,
                              f32, vp]
    lib.pa_decode.restype = i32
    lib.pa_decode_partitioned.argtypes = [vp, i32, vp, vp, vp, i32, vp, i32, vp, i32, i32, i32, i32,
                                          i32, i64, f32, i32, i32, vp, sz, vp]
    lib.pa_decode_partitioned.restype = i32
    lib.pa_decode_balanced.argtypes = [vp, i32, vp, vp, vp, i32, vp, i32, vp, i32, i32, i32, i32,
                                       i32, i64, f32, vp, sz, vp]
    lib.pa_decode_balanced.restype = i32
    lib.pa_decode_step.argtypes = [vp, i32, vp, vp, vp, vp, vp, i32, vp, i32, vp, i32, i32, i32, i32,
                                   i32, i64, f32, vp, sz, vp]
    lib.pa_decode_step.restype = i32
    lib.pa_decode_partitioned_step.argtypes = [vp, i32, vp, vp, vp, vp, vp, i32, vp, i32, vp, i32, i32,
                                               i32, i32, i32, i64, f32, i32, i32, vp, sz, vp]
    lib.pa_decode_partitioned_step.restype = i32
    lib.pa_decode_balanced_workspace_size.argtypes = [i32, i32, i32]
    lib.pa_decode_balanced_workspace_size.restype = sz
    lib.pa_decode_partitioned_noalloc.argtypes = [vp, i32, vp, vp, vp, i32, vp, i32, vp, i32, i32,
                                                  i32, i32, i32, i64, f32, i32, i32, vp]
    lib.pa_decode_partitioned_noalloc.restype = i32
    lib.pa_decode_partitioned_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.pa_decode_partitioned_workspace_size.restype = sz
    lib.pa_decode_cascade.argtypes = [vp, i32, vp, vp, vp, i32, vp, i32, vp, i32, i32, i32, i32,
                                      i32, i64, f32, i32, i32, i32, vp, sz, vp]
    lib.pa_decode_cascade.restype = i32
    lib.pa_decode_cascade_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.pa_decode_cascade_workspace_size.restype = sz
    lib.pa_prefill.argtypes = [vp, i32, vp, vp, vp, i32, vp, i32, vp, vp, i64, i32, i32, i32, i32,
                               i32, i64, f32, i32, vp, sz, vp]
    lib.pa_prefill_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.pa_prefill_workspace_size.restype = sz
    lib.pa_prefill.restype = i32
    lib.pa_bm_create.argtypes = [i64, i32]
    lib.pa_bm_create.restype = vp
    lib.pa_bm_destroy.argtypes = [vp]
    lib.pa_bm_destroy.restype = None
    lib.pa_bm_add_sequence.argtypes = [vp, i64, i32, vp]
    lib.pa_bm_add_sequence.restype = i32
    lib.pa_bm_append_token.argtypes = [vp, i64, vp, vp]
    lib.pa_bm_append_token.restype = i32
    lib.pa_bm_fork.argtypes = [vp, i64, i64]
    lib.pa_bm_fork.restype = i32
    lib.pa_bm_free_sequence.argtypes = [vp, i64]
    lib.pa_bm_free_sequence.restype = i32
    lib.pa_bm_num_free_blocks.argtypes = [vp]
    lib.pa_bm_num_free_blocks.restype = i64
    lib.pa_bm_length.argtypes = [vp, i64]
    lib.pa_bm_length.restype = i64
    lib.pa_bm_block_table.argtypes = [vp, i64, vp, i32, ctypes.c_int32]
    lib.pa_bm_block_table.restype = i64
    lib.pa_status_str.argtypes = [i32]
    lib.pa_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().pa_status_str(int(status)).decode()


def pa_status_str(status: int) -> str:
    return status_str(status)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return PA_F32
    if t == torch.bfloat16:
        return PA_BF16
    raise TypeError(f"unsupported dtype {t}; use float32 or bfloat16")


def _dev(*tensors: torch.Tensor) -> None:
    for t in tensors:
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError("all tensors must be GPU tensors (there is no CPU path)")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _stream(t: torch.Tensor, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return stream.cuda_stream


def _check(status: int, where: str) -> None:
    if status != PA_OK:
        raise PagedAttentionError(status, where)


def pa_reshape_and_cache(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                         value_cache: torch.Tensor, slot_mapping: torch.Tensor,
                         stream: Optional[torch.cuda.Stream] = None) -> None:
    """key/value [T, Hkv, D]; key_cache/value_cache [NB, Hkv, 16, D] (same dtype);
    slot_mapping int64 [T]. Writes in place, asynchronously on the stream."""
    _dev(key, value, key_cache, value_cache, slot_mapping)
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    T, Hkv, D = key.shape
    NB, Hkv2, B, D2 = key_cache.shape
    if (Hkv2, D2) != (Hkv, D) or value.shape != key.shape or value_cache.shape != key_cache.shape:
        raise ValueError("key/value and cache shapes disagree")
    if key.dtype != key_cache.dtype or value.dtype != key.dtype or value_cache.dtype != key.dtype:
        raise TypeError("key, value and caches must share one dtype")
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must have one entry per token")
    rc = load().pa_reshape_and_cache(key.data_ptr(), value.data_ptr(), key_cache.data_ptr(),
                                     value_cache.data_ptr(), slot_mapping.data_ptr(), T, Hkv, D, B,
                                     NB, _dtype_code(key.dtype), _stream(key, stream))
    _check(rc, "pa_reshape_and_cache")


def pa_copy_blocks(key_cache: torch.Tensor, value_cache: torch.Tensor,
                   block_mapping: torch.Tensor, stream: Optional[torch.cuda.Stream] = None) -> None:
    """Copy block block_mapping[i, 0] of both pools onto block block_mapping[i, 1]
    (int64 [N, 2] on the GPU), asynchronously on the stream."""
    _dev(key_cache, value_cache, block_mapping)
    if block_mapping.dtype != torch.int64 or block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise TypeError("block_mapping must be int64 [N, 2]")
    NB, Hkv, B, D = key_cache.shape
    if value_cache.shape != key_cache.shape or value_cache.dtype != key_cache.dtype:
        raise ValueError("key and value pools must share a shape and dtype")
    rc = load().pa_copy_blocks(key_cache.data_ptr(), value_cache.data_ptr(), block_mapping.data_ptr(),
                               block_mapping.shape[0], Hkv, D, B, NB, _dtype_code(key_cache.dtype),
                               _stream(key_cache, stream))
    _check(rc, "pa_copy_blocks")


def pa_swap_blocks(src_key: torch.Tensor, src_value: torch.Tensor, dst_key: torch.Tensor,
                   dst_value: torch.Tensor, block_mapping: torch.Tensor,
                   stream: Optional[torch.cuda.Stream] = None) -> None:
    """Copy block block_mapping[i, 0] of the source pools onto block block_mapping[i, 1] of
    the destination pools (K and V), asynchronously. Each tensor is a GPU tensor or a
    pinned host tensor (torch pin_memory()); block_mapping is int64 [N, 2]. The stream is
    the current stream of the GPU that holds a GPU operand (or of the current GPU)."""
    ts = (src_key, src_value, dst_key, dst_value, block_mapping)
    for t in ts:
        if not isinstance(t, torch.Tensor) or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous tensors")
        if t.device.type != "cuda" and not t.is_pinned():
            raise ValueError("host tensors must be pinned (pin_memory()): the GPU reads them")
    if block_mapping.dtype != torch.int64 or block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise TypeError("block_mapping must be int64 [N, 2]")
    SNB, Hkv, B, D = src_key.shape
    DNB = dst_key.shape[0]
    if src_value.shape != src_key.shape or dst_value.shape != dst_key.shape or \
            dst_key.shape[1:] != src_key.shape[1:]:
        raise ValueError("pools must share their block shape")
    if len({src_key.dtype, src_value.dtype, dst_key.dtype, dst_value.dtype}) != 1:
        raise TypeError("pools must share one dtype")
    gpu = next((t.device for t in ts if t.device.type == "cuda"), None)
    if stream is None:
        stream = torch.cuda.current_stream(gpu)
    rc = load().pa_swap_blocks(src_key.data_ptr(), src_value.data_ptr(), SNB, dst_key.data_ptr(),
                               dst_value.data_ptr(), DNB, block_mapping.data_ptr(),
                               block_mapping.shape[0], Hkv, D, B, _dtype_code(src_key.dtype),
                               stream.cuda_stream)
    _check(rc, "pa_swap_blocks")


def pa_stream_read(src: torch.Tensor, sink: torch.Tensor,
                   stream: Optional[torch.cuda.Stream] = None) -> None:
    """Read every 16-byte word of `src` (a contiguous GPU tensor of a multiple of 16
    bytes) once; sink (uint8 [64 * W] on the GPU, W >= 1 workgroups) receives one
    XOR word per wave. A calibration of the achievable HBM read rate."""
    _dev(src, sink)
    nbytes = src.numel() * src.element_size()
    if nbytes % 16 or sink.dtype != torch.uint8 or sink.dim() != 1 or sink.numel() % 64 or \
            not sink.numel():
        raise ValueError("src must hold a multiple of 16 bytes and sink be uint8 [64 * W]")
    rc = load().pa_stream_read(src.data_ptr(), nbytes // 16, sink.data_ptr(), sink.numel() // 64,
                               _stream(src, stream))
    _check(rc, "pa_stream_read")


def _decode_common(out, query, key_cache, value_cache, block_tables, context_lens):
    _dev(out, query, key_cache, value_cache, block_tables, context_lens)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    S, Hq, D = query.shape
    NB, Hkv, B, D2 = key_cache.shape
    if D2 != D or value_cache.shape != key_cache.shape or out.shape != query.shape:
        raise ValueError("query/out/cache shapes disagree")
    if query.dtype != key_cache.dtype or value_cache.dtype != key_cache.dtype:
        raise TypeError("query and caches must share one dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [S, MB] and context_lens [S]")
    return S, Hq, Hkv, D, B, NB, block_tables.shape[1]


def pa_decode(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
              value_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
              scale: float, stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Single-pass paged decode attention. out [S, Hq, D] (float32 or bfloat16) is written
    asynchronously and returned."""
    S, Hq, Hkv, D, B, NB, MB = _decode_common(out, query, key_cache, value_cache, block_tables,
                                              context_lens)
    rc = load().pa_decode(out.data_ptr(), _dtype_code(out.dtype), query.data_ptr(),
                          key_cache.data_ptr(), value_cache.data_ptr(), _dtype_code(key_cache.dtype),
                          block_tables.data_ptr(), MB, context_lens.data_ptr(), S, Hq, Hkv, D, B,
                          NB, float(scale), _stream(query, stream))
    _check(rc, "pa_decode")
    return out


def pa_prefill_workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                              max_query_len: int) -> int:
    return int(load().pa_prefill_workspace_size(num_seqs, num_q_heads, num_kv_heads, max_query_len))


def pa_prefill(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
               value_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
               query_start: torch.Tensor, scale: float, max_query_len: int,
               workspace: Optional[torch.Tensor] = None,
               stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Multi-token queries over the paged cache. query and out are [T, Hq, D]; the rows of
    sequence s are query_start[s] .. query_start[s + 1] - 1 (int32 [S + 1] on the GPU), the
    last tokens of its context, each attending causally. max_query_len bounds every
    sequence's row count. workspace: a uint8 GPU tensor of pa_prefill_workspace_size()
    bytes (allocated here when None). out (float32 or bfloat16) is written asynchronously
    and returned."""
    _dev(out, query, key_cache, value_cache, block_tables, context_lens, query_start)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32 or \
            query_start.dtype != torch.int32:
        raise TypeError("block_tables, context_lens and query_start must be int32")
    T, Hq, D = query.shape
    NB, Hkv, B, D2 = key_cache.shape
    S = context_lens.shape[0]
    if D2 != D or value_cache.shape != key_cache.shape or out.shape != query.shape:
        raise ValueError("query/out/cache shapes disagree")
    if query.dtype != key_cache.dtype or value_cache.dtype != key_cache.dtype:
        raise TypeError("query and caches must share one dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or query_start.shape != (S + 1,):
        raise ValueError("block_tables must be [S, MB] and query_start [S + 1]")
    if workspace is None:
        n = pa_prefill_workspace_size(S, Hq, Hkv, max(int(max_query_len), 0))
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=query.device)
    _dev(workspace)
    rc = load().pa_prefill(out.data_ptr(), _dtype_code(out.dtype), query.data_ptr(),
                           key_cache.data_ptr(), value_cache.data_ptr(), _dtype_code(key_cache.dtype),
                           block_tables.data_ptr(), block_tables.shape[1], context_lens.data_ptr(),
                           query_start.data_ptr(), T, S, Hq, Hkv, D, B, NB, float(scale),
                           int(max_query_len), workspace.data_ptr(),
                           workspace.numel() * workspace.element_size(), _stream(query, stream))
    _check(rc, "pa_prefill")
    return out


def pa_decode_partitioned_workspace_size(num_seqs: int, num_q_heads: int, head_size: int,
                                         max_context_len: int, partition_size: int) -> int:
    return int(load().pa_decode_partitioned_workspace_size(num_seqs, num_q_heads, head_size,
                                                           max_context_len, partition_size))


def pa_decode_partitioned(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                          value_cache: torch.Tensor, block_tables: torch.Tensor,
                          context_lens: torch.Tensor, scale: float, max_context_len: int,
                          partition_size: int, workspace: torch.Tensor,
                          stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Split-context paged decode attention. workspace is a uint8 GPU tensor of at least
    pa_decode_partitioned_workspace_size(...) bytes (decode_workspace() makes one)."""
    S, Hq, Hkv, D, B, NB, MB = _decode_common(out, query, key_cache, value_cache, block_tables,
                                              context_lens)
    _dev(workspace)
    rc = load().pa_decode_partitioned(out.data_ptr(), _dtype_code(out.dtype), query.data_ptr(),
                                      key_cache.data_ptr(), value_cache.data_ptr(),
                                      _dtype_code(key_cache.dtype), block_tables.data_ptr(), MB,
                                      context_lens.data_ptr(), S, Hq, Hkv, D, B, NB, float(scale),
                                      int(max_context_len), int(partition_size),
                                      workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                      _stream(query, stream))
    _check(rc, "pa_decode_partitioned")
    return out


def pa_decode_balanced_workspace_size(num_q_heads: int, num_kv_heads: int, head_size: int) -> int:
    return int(load().pa_decode_balanced_workspace_size(num_q_heads, num_kv_heads, head_size))


def balanced_workspace(num_q_heads: int, num_kv_heads: int, head_size: int,
                       device=None) -> torch.Tensor:
    """An uninitialised uint8 GPU workspace of the size pa_decode_balanced and
    pa_decode_step need (independent of the batch)."""
    n = pa_decode_balanced_workspace_size(num_q_heads, num_kv_heads, head_size)
    if n == 0:
        raise ValueError("workspace size out of range")
    return torch.empty(n, dtype=torch.uint8, device=device if device is not None else "cuda")


def pa_decode_balanced(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                       value_cache: torch.Tensor, block_tables: torch.Tensor,
                       context_lens: torch.Tensor, scale: float, workspace: torch.Tensor,
                       stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Paged decode attention with the batch's blocks split evenly over the GPU."""
    S, Hq, Hkv, D, B, NB, MB = _decode_common(out, query, key_cache, value_cache, block_tables,
                                              context_lens)
    _dev(workspace)
    rc = load().pa_decode_balanced(out.data_ptr(), _dtype_code(out.dtype), query.data_ptr(),
                                   key_cache.data_ptr(), value_cache.data_ptr(),
                                   _dtype_code(key_cache.dtype), block_tables.data_ptr(), MB,
                                   context_lens.data_ptr(), S, Hq, Hkv, D, B, NB, float(scale),
                                   workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                   _stream(query, stream))
    _check(rc, "pa_decode_balanced")
    return out


def _step_inputs(key, value, key_cache, value_cache, S, Hkv, D, workspace):
    _dev(key, value, workspace)
    if key.shape != (S, Hkv, D) or value.shape != key.shape:
        raise ValueError("key and value must be [S, Hkv, D]")
    if key.dtype != key_cache.dtype or value.dtype != key_cache.dtype:
        raise TypeError("key, value and caches must share one dtype")


def pa_decode_partitioned_step(out: torch.Tensor, query: torch.Tensor, key: torch.Tensor,
                               value: torch.Tensor, key_cache: torch.Tensor,
                               value_cache: torch.Tensor, block_tables: torch.Tensor,
                               context_lens: torch.Tensor, scale: float, max_context_len: int,
                               partition_size: int, workspace: torch.Tensor,
                               stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """One decode step on the partitioned schedule: key/value [S, Hkv, D] (each sequence's
    new token) are written at position context_lens[s] - 1 through the block table, and out
    is the attention over the whole context, new token included. workspace as for
    pa_decode_partitioned (decode_workspace() makes one)."""
    S, Hq, Hkv, D, B, NB, MB = _decode_common(out, query, key_cache, value_cache, block_tables,
                                              context_lens)
    _step_inputs(key, value, key_cache, value_cache, S, Hkv, D, workspace)
    rc = load().pa_decode_partitioned_step(
        out.data_ptr(), _dtype_code(out.dtype), query.data_ptr(), key.data_ptr(), value.data_ptr(),
        key_cache.data_ptr(), value_cache.data_ptr(), _dtype_code(key_cache.dtype),
        block_tables.data_ptr(), MB, context_lens.data_ptr(), S, Hq, Hkv, D, B, NB, float(scale),
        int(max_context_len), int(partition_size), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(query, stream))
    _check(rc, "pa_decode_partitioned_step")
    return out


def pa_decode_step(out: torch.Tensor, query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                   key_cache: torch.Tensor, value_cache: torch.Tensor, block_tables: torch.Tensor,
                   context_lens: torch.Tensor, scale: float, workspace: torch.Tensor,
                   stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """One decode step: key/value [S, Hkv, D] (each sequence's new token) are written at
    position context_lens[s] - 1 through the block table, and out is the attention over the
    whole context, new token included."""
    S, Hq, Hkv, D, B, NB, MB = _decode_common(out, query, key_cache, value_cache, block_tables,
                                              context_lens)
    _step_inputs(key, value, key_cache, value_cache, S, Hkv, D, workspace)
    rc = load().pa_decode_step(out.data_ptr(), _dtype_code(out.dtype), query.data_ptr(),
                               key.data_ptr(), value.data_ptr(), key_cache.data_ptr(),
                               value_cache.data_ptr(), _dtype_code(key_cache.dtype),
                               block_tables.data_ptr(), MB, context_lens.data_ptr(), S, Hq, Hkv, D,
                               B, NB, float(scale), workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), _stream(query, stream))
    _check(rc, "pa_decode_step")
    return out


NOALLOC_WORKSPACE_BYTES = 64 * 1024 * 1024     # PA_NOALLOC_WORKSPACE_BYTES


def pa_decode_partitioned_noalloc(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                                  value_cache: torch.Tensor, block_tables: torch.Tensor,
                                  context_lens: torch.Tensor, scale: float, max_context_len: int,
                                  partition_size: int,
                                  stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """pa_decode_partitioned with its workspace in the library's own per-GPU device buffer
    (NOALLOC_WORKSPACE_BYTES): nothing is allocated. Calls that may overlap in time on one
    GPU race on that buffer."""
    S, Hq, Hkv, D, B, NB, MB = _decode_common(out, query, key_cache, value_cache, block_tables,
                                              context_lens)
    rc = load().pa_decode_partitioned_noalloc(out.data_ptr(), _dtype_code(out.dtype),
                                              query.data_ptr(), key_cache.data_ptr(),
                                              value_cache.data_ptr(), _dtype_code(key_cache.dtype),
                                              block_tables.data_ptr(), MB, context_lens.data_ptr(),
                                              S, Hq, Hkv, D, B, NB, float(scale),
                                              int(max_context_len), int(partition_size),
                                              _stream(query, stream))
    _check(rc, "pa_decode_partitioned_noalloc")
    return out


def pa_decode_cascade_workspace_size(num_seqs: int, num_q_heads: int, head_size: int,
                                     max_context_len: int, partition_size: int,
                                     num_prefix_blocks: int) -> int:
    return int(load().pa_decode_cascade_workspace_size(num_seqs, num_q_heads, head_size,
                                                       max_context_len, partition_size,
                                                       num_prefix_blocks))


def pa_decode_cascade(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                      value_cache: torch.Tensor, block_tables: torch.Tensor,
                      context_lens: torch.Tensor, scale: float, num_prefix_blocks: int,
                      max_context_len: int, partition_size: int, workspace: torch.Tensor,
                      stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Decode attention for a batch whose block tables all start with the same
    num_prefix_blocks ids (read from row 0). workspace is a uint8 GPU tensor of at least
    pa_decode_cascade_workspace_size(...) bytes (cascade_workspace() makes one)."""
    S, Hq, Hkv, D, B, NB, MB = _decode_common(out, query, key_cache, value_cache, block_tables,
                                              context_lens)
    _dev(workspace)
    rc = load().pa_decode_cascade(out.data_ptr(), _dtype_code(out.dtype), query.data_ptr(),
                                  key_cache.data_ptr(), value_cache.data_ptr(),
                                  _dtype_code(key_cache.dtype), block_tables.data_ptr(), MB,
                                  context_lens.data_ptr(), S, Hq, Hkv, D, B, NB, float(scale),
                                  int(num_prefix_blocks), int(max_context_len), int(partition_size),
                                  workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  _stream(query, stream))
    _check(rc, "pa_decode_cascade")
    return out


def cascade_workspace(num_seqs: int, num_q_heads: int, head_size: int, max_context_len: int,
                      partition_size: int, num_prefix_blocks: int, device=None) -> torch.Tensor:
    """An uninitialised uint8 GPU workspace of the size pa_decode_cascade needs."""
    n = pa_decode_cascade_workspace_size(num_seqs, num_q_heads, head_size, max_context_len,
                                         partition_size, num_prefix_blocks)
    if n == 0:
        raise ValueError("workspace size out of range")
    return torch.empty(n, dtype=torch.uint8, device=device if device is not None else "cuda")


def decode_workspace(num_seqs: int, num_q_heads: int, head_size: int, max_context_len: int,
                     partition_size: int, device=None) -> torch.Tensor:
    """An uninitialised uint8 GPU workspace of the size pa_decode_partitioned needs."""
    n = pa_decode_partitioned_workspace_size(num_seqs, num_q_heads, head_size, max_context_len,
                                             partition_size)
    if n == 0:
        raise ValueError("workspace size out of range")
    return torch.empty(n, dtype=torch.uint8, device=device if device is not None else "cuda")


def workspace_partials(workspace: torch.Tensor, num_seqs: int, num_q_heads: int, head_size: int,
                       max_context_len: int, partition_size: int):
    """Views of the partition statistics a pa_decode_partitioned call leaves in its
    workspace: (part_max [S, Hq, NP] natural-log units, part_sum [S, Hq, NP],
    part_out [S, Hq, NP, D]). The layout is the one include/pa.h documents."""
    np_ = max(1, -(-max_context_len // partition_size))
    rows = num_seqs * num_q_heads * np_
    a256 = lambda n: (n + 255) // 256 * 256
    flat = workspace.view(torch.uint8)
    o1 = a256(rows * 4)
    pm = flat[:rows * 4].view(torch.float32).view(num_seqs, num_q_heads, np_)
    ps = flat[o1:o1 + rows * 4].view(torch.float32).view(num_seqs, num_q_heads, np_)
    po = flat[2 * o1:2 * o1 + rows * 4 * head_size].view(torch.float32).view(
        num_seqs, num_q_heads, np_, head_size)
    return pm, ps, po


class NoSpace(PagedAttentionError):
    """The block manager has no free block for the request (nothing changed)."""


class BlockManager:
    """The library's host-side block manager (pa_bm_* in include/pa.h): blocks of the
    pool handed out on demand, per-sequence block tables, shared blocks with reference
    counts, copy-on-write pairs on appends to a shared block."""

    def __init__(self, num_blocks: int, block_size: int = 16):
        self._lib = load()
        self._h = self._lib.pa_bm_create(int(num_blocks), int(block_size))
        if not self._h:
            raise PagedAttentionError(PA_EINVAL, "pa_bm_create")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def _check(self, rc: int, where: str) -> None:
        if rc == PA_ENOSPACE:
            raise NoSpace(rc, where)
        if rc != PA_OK:
            raise PagedAttentionError(rc, where)

    def add_sequence(self, seq: int, num_tokens: int):
        """Blocks for a new sequence; returns the slots of its tokens (list of int)."""
        out = (ctypes.c_int64 * max(1, int(num_tokens)))()
        self._check(self._lib.pa_bm_add_sequence(self._h, int(seq), int(num_tokens), out),
                    "pa_bm_add_sequence")
        return list(out[:int(num_tokens)])

    def append_token(self, seq: int):
        """Room for one more token: (slot, (src, dst) copy-on-write pair or None)."""
        slot = ctypes.c_int64()
        cow = (ctypes.c_int64 * 2)()
        self._check(self._lib.pa_bm_append_token(self._h, int(seq), ctypes.byref(slot), cow),
                    "pa_bm_append_token")
        return slot.value, (None if cow[0] < 0 else (cow[0], cow[1]))

    def fork(self, parent: int, child: int) -> None:
        self._check(self._lib.pa_bm_fork(self._h, int(parent), int(child)), "pa_bm_fork")

    def free_sequence(self, seq: int) -> None:
        self._check(self._lib.pa_bm_free_sequence(self._h, int(seq)), "pa_bm_free_sequence")

    preempt = free_sequence

    def num_free(self) -> int:
        return int(self._lib.pa_bm_num_free_blocks(self._h))

    def length(self, seq: int) -> int:
        n = int(self._lib.pa_bm_length(self._h, int(seq)))
        if n < 0:
            raise PagedAttentionError(PA_EINVAL, "pa_bm_length")
        return n

    def table(self, seq: int, width: int = 0, pad: int = -1):
        """The sequence's block table (list), padded with `pad` to `width` entries if wider."""
        n = int(self._lib.pa_bm_block_table(self._h, int(seq), None, 0, 0))
        if n < 0:
            raise PagedAttentionError(PA_EINVAL, "pa_bm_block_table")
        w = max(n, int(width))
        buf = (ctypes.c_int32 * max(1, w))()
        self._lib.pa_bm_block_table(self._h, int(seq), buf, w, int(pad))
        return list(buf[:w])

"""fp64 CPU oracle for paged decode attention, multi-token queries over the paged
cache, the KV-cache write, the copy-on-write block copy and the block swap between
two pools (the block manager's reference model is the plain Python of
``block_manager.py``).

TEST INFRASTRUCTURE ONLY. The test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers. The GPU library never
imports, links or runs anything in this directory, and this directory never
imports the GPU package.

The arithmetic lives in ``pa_oracle.c`` (plain C, fp64, loops that follow the
definitions; its header states them and where the pages support them). This
module only builds that library with gcc, converts inputs to fp64 arrays
(exactly: bf16 and fp32 values are representable in fp64) and calls it.

Parity status: every function here is pinned by ``tests/test_oracle.py``
(library routine, brute force, closed forms and invariants). The pages print
no attention values, so beyond those pins the oracle is the definition.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libpa_oracle.so")
_LIB = None

_ERRORS = {
    -1: "invalid argument",
    -2: "block table entry outside the pool",
    -3: "context length negative or beyond the block table / partitions",
    -4: "slot past the end of the pool",
    -5: "two tokens write the same slot",
    -6: "out of memory",
    -7: "block copy past the pool, or whose result would depend on the copy order",
}


class OracleError(RuntimeError):
    pass


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (-O2, OpenMP). Returns the library path."""
    cmd = ["gcc", "-O2", "-fopenmp", "-std=c99", "-shared", "-fPIC", "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str = _LIB_PATH) -> ctypes.CDLL:
    lib = ctypes.CDLL(path)
    i32p = ctypes.POINTER(ctypes.c_int32)
    i64p = ctypes.POINTER(ctypes.c_int64)
    dp = ctypes.POINTER(ctypes.c_double)
    u8p = ctypes.c_void_p
    lib.oracle_reshape_and_cache.argtypes = [u8p, u8p, u8p, u8p, i64p, ctypes.c_int64,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int64, ctypes.c_int]
    lib.oracle_reshape_and_cache.restype = ctypes.c_int
    lib.oracle_decode.argtypes = [dp, dp, dp, dp, i32p, i32p, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int64, ctypes.c_double, ctypes.c_int]
    lib.oracle_decode.restype = ctypes.c_int
    lib.oracle_decode_partitioned.argtypes = [dp, dp, dp, dp, dp, dp, dp, i32p, i32p,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int64, ctypes.c_double, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int]
    lib.oracle_decode_partitioned.restype = ctypes.c_int
    lib.oracle_prefill.argtypes = [dp, dp, dp, dp, i32p, i32p, i32p, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int64, ctypes.c_double, ctypes.c_int]
    lib.oracle_prefill.restype = ctypes.c_int
    lib.oracle_copy_blocks.argtypes = [u8p, u8p, i64p, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int64]
    lib.oracle_copy_blocks.restype = ctypes.c_int
    lib.oracle_swap_blocks.argtypes = [u8p, u8p, ctypes.c_int64, u8p, u8p, ctypes.c_int64, i64p,
                                       ctypes.c_int64, ctypes.c_int64]
    lib.oracle_swap_blocks.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _LIB = load()
    return _LIB


def max_threads() -> int:
    return int(_lib().oracle_max_threads())


def _f64(x) -> np.ndarray:
    """Exact conversion of a numpy array or torch CPU tensor to a C-contiguous fp64 array."""
    if hasattr(x, "detach"):           # torch tensor (bf16 has no numpy dtype)
        import torch
        return np.ascontiguousarray(x.detach().to("cpu", torch.float64).numpy())
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i32(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _check(rc: int) -> None:
    if rc != 0:
        raise OracleError(_ERRORS.get(rc, f"oracle error {rc}"))


def fp32_scale(scale: float) -> float:
    """The scale the GPU library receives is a C float; the oracle uses that exact value."""
    return float(np.float32(scale))


def reshape_and_cache(key: np.ndarray, value: np.ndarray, key_cache: np.ndarray,
                      value_cache: np.ndarray, slot_mapping, block_size: int = 16,
                      lib: Optional[ctypes.CDLL] = None) -> None:
    """Write each new token's K and V into its slot, in place, byte for byte.

    key, value:              [T, Hkv, D] numpy arrays (any dtype; bf16 as uint16 views)
    key_cache, value_cache:  [NB, Hkv, B, D] numpy arrays of the same dtype, C-contiguous
    slot_mapping:            [T] int64; a negative slot skips its token
    """
    lib = lib or _lib()
    for a in (key, value, key_cache, value_cache):
        if not a.flags["C_CONTIGUOUS"]:
            raise ValueError("arrays must be C-contiguous")
    if key.dtype != key_cache.dtype or value.dtype != value_cache.dtype:
        raise ValueError("new tokens and cache must share a dtype")
    slots = np.ascontiguousarray(np.asarray(slot_mapping, dtype=np.int64))
    T, Hkv, D = key.shape
    NB = key_cache.shape[0]
    if key_cache.shape != (NB, Hkv, block_size, D) or value_cache.shape != key_cache.shape:
        raise ValueError("cache shape must be [NB, Hkv, block_size, D]")
    if value.shape != key.shape or slots.shape != (T,):
        raise ValueError("key/value/slot_mapping shapes disagree")
    rc = lib.oracle_reshape_and_cache(key.ctypes.data, value.ctypes.data, key_cache.ctypes.data,
                                      value_cache.ctypes.data, _ptr(slots, ctypes.c_int64),
                                      T, Hkv, D, block_size, NB, key.dtype.itemsize)
    _check(rc)


def copy_blocks(key_cache: np.ndarray, value_cache: np.ndarray, block_mapping,
                lib: Optional[ctypes.CDLL] = None) -> None:
    """Copy-on-write block copy, in place, byte for byte: for each pair (src, dst) of
    block_mapping ([N, 2] int64), block dst of both pools becomes a copy of block src.
    Pools are [NB, Hkv, B, D] numpy arrays (bf16 as uint16 views), C-contiguous."""
    lib = lib or _lib()
    for a in (key_cache, value_cache):
        if not a.flags["C_CONTIGUOUS"]:
            raise ValueError("arrays must be C-contiguous")
    if key_cache.shape != value_cache.shape or key_cache.dtype != value_cache.dtype:
        raise ValueError("pools must share a shape and dtype")
    pairs = np.ascontiguousarray(np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2))
    NB = key_cache.shape[0]
    block_bytes = key_cache.nbytes // NB if NB else 1
    rc = lib.oracle_copy_blocks(key_cache.ctypes.data, value_cache.ctypes.data,
                                _ptr(pairs, ctypes.c_int64), pairs.shape[0], block_bytes, NB)
    _check(rc)


def swap_blocks(src_key: np.ndarray, src_value: np.ndarray, dst_key: np.ndarray,
                dst_value: np.ndarray, block_mapping, lib: Optional[ctypes.CDLL] = None) -> None:
    """Block swap between two pairs of pools, byte for byte: for each pair (src, dst) of
    block_mapping ([N, 2] int64), block dst of the destination pools becomes a copy of
    block src of the source pools (both K and V). Pools are [NB, Hkv, B, D] numpy arrays
    (bf16 as uint16 views), C-contiguous; source and destination may differ in NB only.
    The destination arrays are written in place."""
    lib = lib or _lib()
    for a in (src_key, src_value, dst_key, dst_value):
        if not a.flags["C_CONTIGUOUS"]:
            raise ValueError("arrays must be C-contiguous")
    if src_key.shape != src_value.shape or dst_key.shape != dst_value.shape or \
            src_key.shape[1:] != dst_key.shape[1:] or \
            len({src_key.dtype, src_value.dtype, dst_key.dtype, dst_value.dtype}) != 1:
        raise ValueError("pools must share a block shape and dtype")
    pairs = np.ascontiguousarray(np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2))
    block_bytes = int(np.prod(src_key.shape[1:])) * src_key.itemsize
    rc = lib.oracle_swap_blocks(src_key.ctypes.data, src_value.ctypes.data, src_key.shape[0],
                                dst_key.ctypes.data, dst_value.ctypes.data, dst_key.shape[0],
                                _ptr(pairs, ctypes.c_int64), pairs.shape[0], block_bytes)
    _check(rc)


def decode(query, key_cache, value_cache, block_tables, context_lens, scale: float,
           num_threads: int = 0, lib: Optional[ctypes.CDLL] = None) -> np.ndarray:
    """Single-pass decode attention in fp64. Returns out [S, Hq, D] (float64).

    query [S, Hq, D]; key_cache/value_cache [NB, Hkv, B, D]; block_tables [S, MB] int32;
    context_lens [S] int32; scale is rounded to fp32 first, as the GPU library receives it.
    """
    lib = lib or _lib()
    q = _f64(query)
    kc = _f64(key_cache)
    vc = _f64(value_cache)
    bt = _i32(block_tables)
    cl = _i32(context_lens)
    S, Hq, D = q.shape
    NB, Hkv, B, D2 = kc.shape
    if D2 != D or vc.shape != kc.shape or bt.shape[0] != S or cl.shape != (S,):
        raise ValueError("shapes disagree")
    out = np.zeros((S, Hq, D), dtype=np.float64)
    rc = lib.oracle_decode(_ptr(out, ctypes.c_double), _ptr(q, ctypes.c_double),
                           _ptr(kc, ctypes.c_double), _ptr(vc, ctypes.c_double),
                           _ptr(bt, ctypes.c_int32), _ptr(cl, ctypes.c_int32),
                           S, Hq, Hkv, D, B, bt.shape[1], NB, fp32_scale(scale), num_threads)
    _check(rc)
    return out


def decode_partitioned(query, key_cache, value_cache, block_tables, context_lens, scale: float,
                       partition_size: int, num_partitions: Optional[int] = None,
                       num_threads: int = 0, lib: Optional[ctypes.CDLL] = None
                       ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Split-context decode in fp64. Returns (out, part_max, part_sum, part_out) with
    part_max/part_sum [S, Hq, NP] and part_out [S, Hq, NP, D]; part_max is in natural-log
    units of the scaled logits."""
    lib = lib or _lib()
    q = _f64(query)
    kc = _f64(key_cache)
    vc = _f64(value_cache)
    bt = _i32(block_tables)
    cl = _i32(context_lens)
    S, Hq, D = q.shape
    NB, Hkv, B, _ = kc.shape
    if num_partitions is None:
        num_partitions = max(1, -(-int(cl.max(initial=0)) // partition_size))
    out = np.zeros((S, Hq, D), dtype=np.float64)
    pm = np.zeros((S, Hq, num_partitions), dtype=np.float64)
    ps = np.zeros((S, Hq, num_partitions), dtype=np.float64)
    po = np.zeros((S, Hq, num_partitions, D), dtype=np.float64)
    rc = lib.oracle_decode_partitioned(
        _ptr(out, ctypes.c_double), _ptr(pm, ctypes.c_double), _ptr(ps, ctypes.c_double),
        _ptr(po, ctypes.c_double), _ptr(q, ctypes.c_double), _ptr(kc, ctypes.c_double),
        _ptr(vc, ctypes.c_double), _ptr(bt, ctypes.c_int32), _ptr(cl, ctypes.c_int32),
        S, Hq, Hkv, D, B, bt.shape[1], NB, fp32_scale(scale), partition_size, num_partitions,
        num_threads)
    _check(rc)
    return out, pm, ps, po


def prefill(query, key_cache, value_cache, block_tables, context_lens, query_start, scale: float,
            num_threads: int = 0, lib: Optional[ctypes.CDLL] = None) -> np.ndarray:
    """Multi-token queries over the paged cache in fp64. Returns out [T, Hq, D] (float64).

    query [T, Hq, D] with T = query_start[-1]; query_start [S + 1] int32 (0, then
    non-decreasing): the rows of sequence s are query_start[s] .. query_start[s + 1] - 1, the
    last q_s tokens of its context, and row i attends causally to tokens
    0 .. context_lens[s] - q_s + i.
    """
    lib = lib or _lib()
    q = _f64(query)
    kc = _f64(key_cache)
    vc = _f64(value_cache)
    bt = _i32(block_tables)
    cl = _i32(context_lens)
    qs = _i32(query_start)
    T, Hq, D = q.shape
    NB, Hkv, B, D2 = kc.shape
    S = cl.shape[0]
    if D2 != D or vc.shape != kc.shape or bt.shape[0] != S or qs.shape != (S + 1,) or \
            (S > 0 and int(qs[-1]) != T):
        raise ValueError("shapes disagree")
    out = np.zeros((T, Hq, D), dtype=np.float64)
    rc = lib.oracle_prefill(_ptr(out, ctypes.c_double), _ptr(q, ctypes.c_double),
                            _ptr(kc, ctypes.c_double), _ptr(vc, ctypes.c_double),
                            _ptr(bt, ctypes.c_int32), _ptr(cl, ctypes.c_int32),
                            _ptr(qs, ctypes.c_int32), S, Hq, Hkv, D, B, bt.shape[1], NB,
                            fp32_scale(scale), num_threads)
    _check(rc)
    return out

"""Seeded synthetic inputs for paged decode attention.

This module builds the inputs of one decode step: the query of each running
sequence, the two physical KV block pools, the per-sequence block tables,
the context lengths, and the new tokens with their slot mapping. It is shared
by the CPU oracle tests, the GPU parity tests and the benchmark, and it holds
none of the attention arithmetic: it only draws numbers and lays them out.

Conventions (the pages give the idea, not a layout; these are the readings
used throughout):

* A KV block holds 16 tokens ("Idea 1: PagedAttention" on the day-9 post of
  skandtandon.pages.dev says blocks are typically 16 tokens).
* Each pool is ``[num_blocks, num_kv_heads, block_size, head_size]``; one
  physical block id addresses every KV head.
* ``block_tables[s, j]`` is the physical block of logical block ``j`` of
  sequence ``s`` (the block table of "The idea vLLM started from: pages" on
  "What vLLM Is and Why It Exists"). Entries past ``ceil(L_s / 16)`` are
  padding and are never read.
* The token just produced by a sequence is part of its context: it is token
  ``L_s - 1`` and lives in slot ``block * 16 + offset`` of the pool.
* Physical blocks are handed out as a seeded random permutation of the free
  blocks, so logically adjacent blocks are scattered through the pool.

Values are N(0, 1) draws cast to the workload dtype. Memory the kernels must
not read (unused blocks, the tail of each sequence's last block, the slots
that the cache write is about to fill) is poisoned with NaN so that a stray
read shows up in the output.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np
import torch

BLOCK_SIZE = 16

# Per-workload seeds: values use 1000 + index, lengths and tables 2000 + index.
_VALUE_SEED_BASE = 1000
_LAYOUT_SEED_BASE = 2000


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    """Shape and length law of one synthetic decode workload."""

    index: int
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_size: int
    dtype: torch.dtype
    lengths: str                 # how context lengths are drawn (see _draw_lengths)
    pool: str                    # how the physical pool is sized (see _pool_blocks)
    new_tokens_per_seq: int = 1
    partition_size: int = 512
    description: str = ""


SPECS: Dict[str, WorkloadSpec] = {
    "tiny_fp32": WorkloadSpec(
        0, "tiny_fp32", num_seqs=4, num_q_heads=4, num_kv_heads=4, head_size=64,
        dtype=torch.float32, lengths="fixed:1,15,16,37", pool="fixed:32",
        partition_size=32,
        description="4 sequences with context lengths 1/15/16/37, 4 query heads = 4 KV "
                    "heads, head size 64, fp32, pool of 32 blocks"),
    "llama8b_gqa_bf16": WorkloadSpec(
        1, "llama8b_gqa_bf16", num_seqs=64, num_q_heads=32, num_kv_heads=8, head_size=128,
        dtype=torch.bfloat16, lengths="exp:100,400,4096", pool="twice",
        partition_size=256,
        description="Llama-8B-shaped GQA decode: 64 sequences, 32 query / 8 KV heads, head "
                    "size 128, bf16, L = min(4096, 100 + floor(Exp(mean 400))), pool 2x needed"),
    "large_batch_bf16": WorkloadSpec(
        2, "large_batch_bf16", num_seqs=256, num_q_heads=32, num_kv_heads=8, head_size=128,
        dtype=torch.bfloat16, lengths="uniform:1024,8192", pool="hbm:0.6",
        partition_size=512,
        description="256 sequences, 32 query / 8 KV heads, head size 128, bf16, L uniform in "
                    "[1024, 8192], pool sized to 60% of 288 GB"),
    "prefix_shared_bf16": WorkloadSpec(
        3, "prefix_shared_bf16", num_seqs=128, num_q_heads=32, num_kv_heads=8, head_size=128,
        dtype=torch.bfloat16, lengths="prefix:2048,1,512", pool="twice",
        partition_size=256,
        description="128 sequences sharing 128 physical prefix blocks (2048 tokens), each with "
                    "a private suffix of uniform [1, 512] tokens whose last block is a "
                    "copy-on-write duplicate of a common parent block"),
    "long_context_bf16": WorkloadSpec(
        4, "long_context_bf16", num_seqs=8, num_q_heads=64, num_kv_heads=8, head_size=128,
        dtype=torch.bfloat16, lengths="fixed:32768x8", pool="twice",
        new_tokens_per_seq=8, partition_size=512,
        description="8 sequences x 32768 tokens, 64 query / 8 KV heads, head size 128, bf16, "
                    "512-token partitions, 8 new tokens per sequence"),
}

HBM_BYTES = 288e9


@dataclasses.dataclass
class Workload:
    """One decode step's inputs. Host-side layout arrays are numpy; tensors live on `device`."""

    spec: WorkloadSpec
    num_blocks: int
    block_size: int
    context_lens: np.ndarray        # int32 [S]
    block_tables: np.ndarray        # int32 [S, max_blocks_per_seq]
    slot_mapping: np.ndarray        # int64 [T]; -1 = padding token
    used_blocks: np.ndarray         # int64, every physical block some table reaches
    query: torch.Tensor             # [S, Hq, D]
    key: torch.Tensor               # [T, Hkv, D] new tokens
    value: torch.Tensor             # [T, Hkv, D]
    key_cache: torch.Tensor         # [NB, Hkv, B, D]
    value_cache: torch.Tensor       # [NB, Hkv, B, D]
    scale: float
    shared_blocks: Optional[np.ndarray] = None   # prefix blocks shared by every table
    cow_parent: Optional[int] = None              # parent block of the copy-on-write copies

    @property
    def num_seqs(self) -> int:
        return self.spec.num_seqs

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if len(self.context_lens) else 0

    def kv_bytes(self) -> int:
        """Bytes of K and V that one decode step must read: sum over sequences of
        L_s * Hkv * D * element size, for K and for V."""
        eb = torch.tensor([], dtype=self.spec.dtype).element_size()
        return int(self.context_lens.astype(np.int64).sum()) * self.spec.num_kv_heads \
            * self.spec.head_size * eb * 2


def _draw_lengths(spec: WorkloadSpec, rng: np.random.Generator) -> np.ndarray:
    kind, _, arg = spec.lengths.partition(":")
    if kind == "fixed":
        if "x" in arg:
            val, cnt = arg.split("x")
            return np.full(int(cnt), int(val), dtype=np.int64)
        return np.array([int(v) for v in arg.split(",")], dtype=np.int64)
    if kind == "exp":
        # The length law of the capacity program on "What vLLM Is and Why It
        # Exists" (section "Code"): 100 plus an exponential draw of mean 400,
        # truncated to an integer, capped at 4096.
        base, mean, cap = (int(v) for v in arg.split(","))
        return exp_lengths(spec.num_seqs, rng, base, mean, cap)
    if kind == "uniform":
        lo, hi = (int(v) for v in arg.split(","))
        return rng.integers(lo, hi + 1, size=spec.num_seqs, dtype=np.int64)
    if kind == "prefix":
        prefix, lo, hi = (int(v) for v in arg.split(","))
        return prefix + rng.integers(lo, hi + 1, size=spec.num_seqs, dtype=np.int64)
    raise ValueError(f"unknown length law {spec.lengths!r}")


def _pool_blocks(spec: WorkloadSpec, needed: int, block_size: int, elem_bytes: int) -> int:
    kind, _, arg = spec.pool.partition(":")
    if kind == "fixed":
        return int(arg)
    if kind == "twice":
        return 2 * needed
    if kind == "hbm":
        # K and V pools together take the given fraction of 288 GB.
        per_block = 2 * spec.num_kv_heads * block_size * spec.head_size * elem_bytes
        return int(float(arg) * HBM_BYTES // per_block)
    raise ValueError(f"unknown pool rule {spec.pool!r}")


def _normal(shape, dtype, gen, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(dtype)


def custom_spec(lengths: List[int], num_q_heads: int, num_kv_heads: int, head_size: int,
                dtype: torch.dtype, new_tokens_per_seq: int = 1, index: int = 100) -> WorkloadSpec:
    """A workload of given context lengths and shapes, with a pool twice the blocks needed."""
    return WorkloadSpec(index, f"custom{index}", num_seqs=len(lengths), num_q_heads=num_q_heads,
                        num_kv_heads=num_kv_heads, head_size=head_size, dtype=dtype,
                        lengths="fixed:" + ",".join(str(int(v)) for v in lengths), pool="twice",
                        new_tokens_per_seq=new_tokens_per_seq)


def make_workload(name, device="cpu", *, poison: bool = True, table_pad: int | str = "poison",
                  num_blocks: Optional[int] = None, lengths: Optional[List[int]] = None,
                  seed_offset: int = 0) -> Workload:
    """Build the named workload (or the one a WorkloadSpec describes).

    device      where the value tensors are drawn and kept (the random stream
                depends on the device, the layout does not).
    poison      fill memory the kernels must not read with NaN.
    table_pad   block-table padding: "poison" (a NaN-filled unused block, if
                any), or an integer such as -1.
    num_blocks  override the pool size (for example when the GPU has less
                free memory than the workload asks for).
    lengths     override the context lengths (same count as num_seqs).
    seed_offset added to both seeds, to draw independent replicas.
    """
    spec = name if isinstance(name, WorkloadSpec) else SPECS[name]
    B = BLOCK_SIZE
    elem_bytes = torch.tensor([], dtype=spec.dtype).element_size()
    lay_rng = np.random.default_rng(_LAYOUT_SEED_BASE + spec.index + 7919 * seed_offset)
    L = np.asarray(lengths, dtype=np.int64) if lengths is not None else _draw_lengths(spec, lay_rng)
    if len(L) != spec.num_seqs:
        raise ValueError("lengths must have one entry per sequence")
    S, Hq, Hkv, D = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_size
    nblk = (L + B - 1) // B

    shared = None
    cow_parent = None
    if spec.lengths.startswith("prefix"):
        prefix_blocks = int(spec.lengths.split(":")[1].split(",")[0]) // B
        private = nblk - prefix_blocks
        needed = prefix_blocks + int(private.sum()) + 1        # + the copy-on-write parent
    else:
        needed = int(nblk.sum())
    NB = num_blocks if num_blocks is not None else _pool_blocks(spec, needed, B, elem_bytes)
    if NB < needed + (1 if (poison and table_pad == "poison") else 0):
        raise ValueError(f"pool of {NB} blocks cannot hold {needed} needed blocks")

    # Hand out physical blocks as a seeded random draw of distinct free blocks.
    if NB <= 4_000_000:
        order = lay_rng.permutation(NB)[:needed + 1]
    else:
        order = lay_rng.choice(NB, size=needed + 1, replace=False)
    order = order.astype(np.int64)
    spare = int(order[needed])            # a block no table uses: the poison target
    order = order[:needed]

    MB = int(nblk.max()) if S else 0
    tables = np.zeros((S, max(MB, 1)), dtype=np.int64)
    if spec.lengths.startswith("prefix"):
        shared = order[:prefix_blocks]
        cow_parent = int(order[-1])
        cursor = prefix_blocks
        for s in range(S):
            tables[s, :prefix_blocks] = shared
            n = int(nblk[s]) - prefix_blocks
            tables[s, prefix_blocks:prefix_blocks + n] = order[cursor:cursor + n]
            cursor += n
    else:
        cursor = 0
        for s in range(S):
            n = int(nblk[s])
            tables[s, :n] = order[cursor:cursor + n]
            cursor += n

    pad_value = spare if table_pad == "poison" else int(table_pad)
    for s in range(S):
        tables[s, int(nblk[s]):] = pad_value
    used = np.unique(np.concatenate([tables[s, :int(nblk[s])] for s in range(S)] +
                                    ([np.array([cow_parent])] if cow_parent is not None else [])))

    # New tokens: the last `new_tokens_per_seq` positions of every sequence.
    T_per = spec.new_tokens_per_seq
    slots = []
    for s in range(S):
        for pos in range(int(L[s]) - T_per, int(L[s])):
            if pos < 0:
                slots.append(-1)
                continue
            slots.append(int(tables[s, pos // B]) * B + pos % B)
    slot_mapping = np.asarray(slots, dtype=np.int64)

    # Values.
    gen = torch.Generator(device=device)
    gen.manual_seed(_VALUE_SEED_BASE + spec.index + 7919 * seed_offset)
    dt = spec.dtype
    T = len(slot_mapping)
    query = _normal((S, Hq, D), dt, gen, device)
    key = _normal((T, Hkv, D), dt, gen, device)
    value = _normal((T, Hkv, D), dt, gen, device)

    kc = torch.empty((NB, Hkv, B, D), dtype=dt, device=device)
    vc = torch.empty((NB, Hkv, B, D), dtype=dt, device=device)
    if poison:
        kc.fill_(float("nan"))
        vc.fill_(float("nan"))
    used_t = torch.from_numpy(used).to(device)
    chunk = 1 << 14
    for c0 in range(0, len(used), chunk):
        ids = used_t[c0:c0 + chunk]
        kc.index_copy_(0, ids, _normal((len(ids), Hkv, B, D), dt, gen, device))
        vc.index_copy_(0, ids, _normal((len(ids), Hkv, B, D), dt, gen, device))

    if cow_parent is not None:
        # Copy-on-write: every sequence's last block starts as a copy of the
        # common parent block and diverges from a drawn offset onwards.
        for s in range(S):
            last = int(tables[s, int(nblk[s]) - 1])
            kc[last].copy_(kc[cow_parent])
            vc[last].copy_(vc[cow_parent])
            filled = int(L[s]) - (int(nblk[s]) - 1) * B
            div = int(lay_rng.integers(0, filled))
            n = filled - div
            kc[last, :, div:filled].copy_(_normal((Hkv, n, D), dt, gen, device))
            vc[last, :, div:filled].copy_(_normal((Hkv, n, D), dt, gen, device))

    if poison:
        # Tail slots of every last block, and the slots the cache write fills.
        for s in range(S):
            filled = int(L[s]) - (int(nblk[s]) - 1) * B if L[s] > 0 else 0
            if L[s] > 0 and filled < B:
                last = int(tables[s, int(nblk[s]) - 1])
                kc[last, :, filled:].fill_(float("nan"))
                vc[last, :, filled:].fill_(float("nan"))
        for slot in slot_mapping:
            if slot >= 0:
                kc[slot // B, :, slot % B].fill_(float("nan"))
                vc[slot // B, :, slot % B].fill_(float("nan"))

    return Workload(
        spec=spec, num_blocks=NB, block_size=B,
        context_lens=L.astype(np.int32), block_tables=tables.astype(np.int32),
        slot_mapping=slot_mapping, used_blocks=used,
        query=query, key=key, value=value, key_cache=kc, value_cache=vc,
        scale=1.0 / math.sqrt(D), shared_blocks=shared, cow_parent=cow_parent)


def exp_lengths(n: int, rng: np.random.Generator, base: int = 100, mean: float = 400.0,
                cap: int = 4096) -> np.ndarray:
    """n draws of the skewed length law min(cap, base + floor(Exp(mean)))."""
    draws = np.floor(rng.exponential(mean, size=n)).astype(np.int64)
    return np.minimum(cap, base + draws)


def prefill_queries(w: Workload, query_lens: List[int], seed: int = 0):
    """Query rows for multi-token queries over workload w: sequence s brings the last
    query_lens[s] tokens of its context (each <= its context length). Returns
    (query [T, Hq, D] in the workload dtype, N(0, 1) values drawn on w's device,
    query_start int32 [S + 1] as a numpy array, 0 first)."""
    ql = np.asarray(query_lens, dtype=np.int64)
    if len(ql) != w.num_seqs or (ql < 0).any():
        raise ValueError("one non-negative query length per sequence")
    qs = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    dev = w.key_cache.device
    gen = torch.Generator(device=dev)
    gen.manual_seed(_VALUE_SEED_BASE + 500 + w.spec.index + 7919 * seed)
    q = _normal((int(qs[-1]), w.query.shape[1], w.query.shape[2]), w.query.dtype, gen, dev)
    return q, qs

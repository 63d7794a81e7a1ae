"""Paged KV-cache decode attention for AMD Instinct MI355X (gfx950).

The GPU work lives in ``libpa.so`` (hand-written HIP kernels behind the C-ABI
declared in ``include/pa.h``). This package is its thin Python binding:

    pa_reshape_and_cache   write new tokens' K/V into their cache slots
    pa_copy_blocks         copy whole blocks (copy-on-write)
    pa_swap_blocks         move whole blocks between GPU pools and pinned host pools
    pa_decode              single-pass paged decode attention
    pa_decode_partitioned  split-context decode with a log-sum-exp reduce
    pa_decode_partitioned_noalloc  the same with the library's own per-GPU
                           workspace, for callers that cannot allocate
    pa_decode_balanced     decode with the batch's blocks split evenly over the GPU
    pa_decode_step         the step's cache write and balanced decode in one call
    pa_decode_partitioned_step  the same step on the partitioned schedule
    pa_decode_cascade      decode over a prefix that every sequence shares,
                           read once per KV head, plus per-sequence suffixes
    pa_prefill             multi-token queries (a prompt or a chunk of one)
                           attending causally over the paged cache
    pa_stream_read         streaming-read calibration (the achievable HBM read rate)
    BlockManager           the host-side block manager (pa_bm_*): block tables,
                           shared blocks, copy-on-write pairs
"""
from ._lib import (  # noqa: F401
    PA_BF16, PA_F32, BlockManager, balanced_workspace, pa_decode_balanced,
    pa_decode_balanced_workspace_size, pa_decode_step, NoSpace, PagedAttentionError, cascade_workspace, decode_workspace, load,
    pa_copy_blocks, pa_decode, pa_decode_cascade, pa_decode_cascade_workspace_size,
    pa_decode_partitioned, pa_decode_partitioned_noalloc, pa_decode_partitioned_step,
    pa_decode_partitioned_workspace_size,
    pa_prefill, pa_prefill_workspace_size, pa_reshape_and_cache,
    pa_status_str, pa_stream_read, pa_swap_blocks, workspace_partials,
)

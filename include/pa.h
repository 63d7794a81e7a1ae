/*
 * pa.h -- paged KV-cache decode attention for AMD Instinct MI355X (gfx950).
 *
 * A KV cache cut into fixed-size blocks of 16 tokens, scattered through one
 * shared physical pool and reached through a per-sequence block table
 * ("Idea 1: PagedAttention" on the day-9 post of skandtandon.pages.dev; "The
 * idea vLLM started from: pages" on "What vLLM Is and Why It Exists"; "Paged
 * Attention" on "vLLM Solved the Wrong Bottleneck"). This library provides
 * the two GPU operations of one decode step over such a cache:
 *
 *   pa_reshape_and_cache   write each new token's key and value into its slot
 *   pa_copy_blocks         copy whole blocks (copy-on-write of a shared block)
 *   pa_swap_blocks         move whole blocks between the GPU pools and host
 *                          pools (swap a preempted sequence out and back in)
 *   pa_decode              one query token per sequence attends over its
 *                          block-scattered context (single pass)
 *   pa_decode_partitioned  the same result, with each context cut into
 *                          fixed-size partitions that run in parallel and a
 *                          log-sum-exp reduce across partitions
 *   pa_decode_balanced     the same result with the work cut into equal
 *                          byte ranges over the whole batch
 *   pa_decode_step         cache write of each sequence's new token plus
 *                          balanced decode, in one call
 *   pa_decode_partitioned_step
 *                          the same step on the partitioned schedule
 *   pa_decode_cascade      the same result for a batch whose tables all begin
 *                          with the same physical blocks (a shared prefix):
 *                          the prefix is read once per KV head for the whole
 *                          batch instead of once per sequence
 *
 * Conventions shared by every call
 * --------------------------------
 *  S    num_seqs            Hq  num_q_heads         Hkv num_kv_heads
 *  D    head_size (64 or 128)                       B   block_size (must be 16)
 *  NB   num_blocks in each pool                     MB  max_blocks_per_seq
 *
 *  key_cache, value_cache  [NB][Hkv][B][D], row-major, dtype kv_dtype. One
 *                          physical block id addresses every KV head; the
 *                          (block, head) tile is B*D contiguous elements.
 *  block_tables            int32 [S][MB]: entry [s][j] is the physical block
 *                          holding tokens 16j .. 16j+15 of sequence s. Only
 *                          entries j < ceil(context_lens[s] / 16) are read.
 *  context_lens            int32 [S]: tokens of context of each sequence,
 *                          including the token written in this step.
 *  query, out              [S][Hq][D]. Query head h reads KV head
 *                          h / (Hq / Hkv) (grouped-query attention).
 *  scale                   multiplies q.k before the softmax (typically
 *                          1/sqrt(D)).
 *
 *  The attention computed, per sequence s and query head h, over the tokens
 *  t < L = context_lens[s] (the pages give no formula; this is standard
 *  scaled dot-product softmax attention of the new token over its context):
 *      l_t = scale * q[s][h] . K_t,   w_t = softmax_t(l_t),   out = sum_t w_t V_t
 *  Accumulation is fp32 everywhere (bf16 inputs are exact in fp32). In the
 *  decode calls the softmax weights P stay fp32 through P.V. The dense-tile
 *  calls (the shared-prefix part of pa_decode_cascade, and pa_prefill) run
 *  P.V on bf16 matrix cores with P split into a bf16 high part plus the bf16
 *  rounding of the remainder, which keeps about 16 bits of each weight; their
 *  weights are taken relative to a running reference maximum that moves only
 *  when a logit exceeds it by 8 (base 2), so a weight is at most 256 before
 *  the final normalisation (the same result in exact arithmetic).
 *  L = 0 gives a zero row.
 *
 *  Pointers.   All data pointers are DEVICE pointers, 16-byte aligned, owned
 *              by the caller and kept alive until the work on `stream` has
 *              finished. No call allocates memory and none keeps a pointer
 *              after it returns; the library caches each device's CU count,
 *              LDS size and kernel occupancies on first use, and
 *              pa_decode_partitioned_noalloc uses a workspace array the
 *              library holds on each GPU for the life of the process. Calls
 *              are thread-safe. `out` and `workspace` must not overlap any
 *              input.
 *  Streams.    `stream` is a hipStream_t (NULL = the default stream). Every
 *              call only enqueues work and returns; nothing synchronises.
 *  Errors.     Host-side checks run before anything is enqueued and return:
 *                PA_EINVAL        null or misaligned pointer, negative count,
 *                                 Hq not a multiple of Hkv, bad partition size
 *                PA_EUNSUPPORTED  B != 16, D not 64 or 128, Hq/Hkv > 16,
 *                                 an unsupported dtype
 *                PA_EWORKSPACE    workspace smaller than required
 *                PA_EHIP          the kernel launch failed
 *                PA_ENOSPACE      (block manager) no free block for the request
 *              Device-resident inputs are not copied to the host. The kernels
 *              check them anyway and never touch memory outside the pools:
 *              a sequence whose context is longer than its table (16 * MB
 *              tokens) or, in the partitioned calls, longer than
 *              ceil(max_context_len / partition_size) * partition_size tokens,
 *              or whose table reaches a block id outside [0, NB), gets an
 *              all-NaN output row; a slot outside the pool is skipped by the
 *              cache write.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype_t;

typedef enum {
    PA_OK = 0,
    PA_EINVAL = 1,
    PA_EUNSUPPORTED = 2,
    PA_EWORKSPACE = 3,
    PA_EHIP = 4,
    PA_ENOSPACE = 5
} pa_status_t;

/*
 * pa_reshape_and_cache -- write new tokens' K and V into their slots.
 *
 * The pages say each request keeps the key/value state of every token it has
 * produced ("The problem a naive server has", point 3, on "What vLLM Is and
 * Why It Exists") and holds only the blocks those tokens fill ("The idea vLLM
 * started from: pages"). Slot numbering is a reading: slot = block * 16 +
 * row, so token i lands in key_cache[slot / 16][h][slot % 16][:] for every
 * KV head h.
 *
 *   key, value          [T][Hkv][D] of kv_dtype, T = num_tokens
 *   key_cache, value_cache  the pools, updated in place
 *   slot_mapping        int64 [T]; a negative slot marks a padding token and
 *                       is skipped. Two tokens must not name the same slot.
 *   num_blocks          NB; slots >= NB * 16 are skipped.
 *
 * The copy is bit-exact (no conversion: input dtype = cache dtype).
 * num_tokens = 0 is valid and enqueues nothing.
 */
pa_status_t pa_reshape_and_cache(const void* key, const void* value,
                                 void* key_cache, void* value_cache,
                                 const int64_t* slot_mapping, int64_t num_tokens,
                                 int num_kv_heads, int head_size, int block_size,
                                 int64_t num_blocks, pa_dtype_t kv_dtype, void* stream);

/*
 * pa_copy_blocks -- copy whole blocks within the pools (copy-on-write).
 *
 * When a block shared by several sequences must diverge, only that block is
 * copied ("Idea 1: PagedAttention" on the day-9 post, "Why this wins"). For
 * each pair i, block block_mapping[2i] of both pools (every KV head, every
 * row) is copied onto block block_mapping[2i + 1], byte for byte.
 *
 *   block_mapping  int64 [num_pairs][2] (source, destination), device memory.
 *                  A pair with a negative id, or an id >= num_blocks, is
 *                  skipped. Destinations must be distinct and must not be the
 *                  source of any pair: the copies run in parallel, in no order.
 *   key_cache, value_cache  [NB][Hkv][16][D] of kv_dtype, updated in place.
 *
 * num_pairs = 0 is valid and enqueues nothing.
 */
pa_status_t pa_copy_blocks(void* key_cache, void* value_cache, const int64_t* block_mapping,
                           int64_t num_pairs, int num_kv_heads, int head_size, int block_size,
                           int64_t num_blocks, pa_dtype_t kv_dtype, void* stream);

/*
 * pa_swap_blocks -- move whole blocks between two pairs of pools, typically
 * the GPU pools and a pair of pools in pinned host memory (swap out a
 * preempted sequence, later swap it back in).
 *
 * "Preemption" takes a request's blocks away to feed another ("Why read its
 * source at all" on "What vLLM Is and Why It Exists"); keeping those blocks'
 * contents in host memory lets the request resume without recomputing them.
 * For each pair i, block block_mapping[2i] of the source pools (every KV head,
 * every row, K and V) is copied onto block block_mapping[2i + 1] of the
 * destination pools, byte for byte. Swap-in after swap-out returns the same
 * bytes, so a table remapped to the new blocks decodes bit-identically.
 *
 *   src_key_cache, src_value_cache  [src_num_blocks][Hkv][16][D] of kv_dtype
 *   dst_key_cache, dst_value_cache  [dst_num_blocks][Hkv][16][D], written
 *   block_mapping  int64 [num_pairs][2] (source id, destination id). A pair
 *                  with a negative id, or an id past its own pool, is
 *                  skipped. Destination ids must be distinct.
 * Every pointer is memory the GPU can address: device memory, or pinned host
 * memory (hipHostMalloc; torch's pin_memory()), which the kernel reads or
 * writes across the host link. Pageable host memory gives PA_EINVAL. Source
 * and destination pools must not overlap. The call is asynchronous on
 * `stream`: host pools must stay allocated and untouched until it finishes.
 * num_pairs = 0 is valid and enqueues nothing.
 */
pa_status_t pa_swap_blocks(const void* src_key_cache, const void* src_value_cache,
                           int64_t src_num_blocks, void* dst_key_cache, void* dst_value_cache,
                           int64_t dst_num_blocks, const int64_t* block_mapping, int64_t num_pairs,
                           int num_kv_heads, int head_size, int block_size, pa_dtype_t kv_dtype,
                           void* stream);

/*
 * pa_decode -- single-pass paged decode attention.
 *
 * Reads each sequence's KV cache from blocks scattered through the pools,
 * following its block table ("The idea vLLM started from: pages", "What vLLM
 * Is and Why It Exists"). One workgroup per (sequence, KV head) walks the
 * whole context, so this suits short contexts; long contexts should use
 * pa_decode_partitioned.
 *
 *   out        [S][Hq][D] of out_dtype (PA_F32 or PA_BF16)
 *   query      [S][Hq][D] of kv_dtype
 *   kv_dtype   PA_F32 or PA_BF16, for query, key_cache and value_cache
 *   num_blocks NB, used to reject out-of-pool table entries on the device
 *   num_seqs = 0 is valid and enqueues nothing.
 */
pa_status_t pa_decode(void* out, pa_dtype_t out_dtype, const void* query,
                      const void* key_cache, const void* value_cache, pa_dtype_t kv_dtype,
                      const int32_t* block_tables, int max_blocks_per_seq,
                      const int32_t* context_lens, int num_seqs, int num_q_heads,
                      int num_kv_heads, int head_size, int block_size, int64_t num_blocks,
                      float scale, void* stream);

/*
 * Workspace bytes pa_decode_partitioned needs. With
 * NP = max(1, ceil(max_context_len / partition_size)) and R = S * Hq * NP,
 * the workspace holds three float32 arrays, each starting on a 256-byte
 * boundary: part_max [R], part_sum [R], part_out [R][D], so the size is
 *     2 * round_up(4 R, 256) + round_up(4 R D, 256).
 * Returns 0 when an argument is out of range.
 */
size_t pa_decode_partitioned_workspace_size(int num_seqs, int num_q_heads, int head_size,
                                            int max_context_len, int partition_size);

/*
 * pa_decode_partitioned -- split-context paged decode attention.
 *
 * Same inputs and result as pa_decode. Each context is cut into partitions of
 * partition_size tokens (a multiple of 16); partition p covers tokens
 * [p * partition_size, min((p + 1) * partition_size, L)). Each (sequence,
 * KV head, partition) item -- taken by one wave of a grid of resident
 * workgroups, or by one workgroup when S > 4096 or the batch's context
 * lengths do not fit a workgroup's LDS -- computes the partition's maximum scaled
 * logit m_p, sum s_p = sum exp(l_t - m_p) and normalised partial output o_p;
 * a second kernel combines the partitions of each (sequence, KV head), in
 * partition order:
 *     M = max_p m_p,  w_p = s_p * exp(m_p - M),  out = sum_p w_p o_p / sum_p w_p.
 * (The pages do not describe this variant; it is the standard log-sum-exp
 * split of softmax and equals the single pass in exact arithmetic.)
 * A sequence whose context fits one partition gets its output row written
 * directly, and when every context fits one partition (NP = 1) the second
 * kernel is not launched.
 *
 *   max_context_len  an upper bound on every context_lens[s], known on the
 *                    host; it sizes the grid and the workspace. A context
 *                    longer than ceil(max_context_len / partition_size) *
 *                    partition_size tokens gives a NaN row (one a little
 *                    over max_context_len but within that many partitions is
 *                    still computed).
 *   partition_size   tokens per partition, a positive multiple of 16.
 *   workspace        device scratch of at least
 *                    pa_decode_partitioned_workspace_size(...) bytes, 256-byte
 *                    aligned, laid out as float32 part_max [S][Hq][NP]
 *                    (natural-log units), part_sum [S][Hq][NP] and part_out
 *                    [S][Hq][NP][D] (see the size function). Its contents
 *                    before the call do not matter. After the call, for every
 *                    sequence with more than one partition, the entries of
 *                    partitions p < ceil(L / partition_size) hold the
 *                    partials; all other entries are unspecified.
 */
pa_status_t pa_decode_partitioned(void* out, pa_dtype_t out_dtype, const void* query,
                                  const void* key_cache, const void* value_cache,
                                  pa_dtype_t kv_dtype, const int32_t* block_tables,
                                  int max_blocks_per_seq, const int32_t* context_lens,
                                  int num_seqs, int num_q_heads, int num_kv_heads,
                                  int head_size, int block_size, int64_t num_blocks,
                                  float scale, int max_context_len, int partition_size,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_partitioned_noalloc -- pa_decode_partitioned for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, and harnesses that forbid hipMalloc.
 *
 * Same arguments and result as pa_decode_partitioned, without the workspace
 * arguments: the split's partials live in a buffer of
 * PA_NOALLOC_WORKSPACE_BYTES that the library holds in device memory, one per
 * GPU it runs on, from the first call on that GPU until the process ends.
 * The call allocates and frees nothing (no hipMalloc, no allocating library
 * routine) and, like every call here, only enqueues work on `stream`.
 *
 *   PA_EWORKSPACE  pa_decode_partitioned_workspace_size(num_seqs, num_q_heads,
 *                  head_size, max_context_len, partition_size) exceeds
 *                  PA_NOALLOC_WORKSPACE_BYTES (nothing is enqueued).
 *   PA_EHIP        the buffer's device address could not be obtained.
 *   Other checks and status codes are those of pa_decode_partitioned.
 *
 * Every call on one GPU uses that GPU's single buffer: two calls whose work
 * may overlap in time on the same GPU (different streams, or host threads
 * without ordering) race on it and give undefined results. Calls ordered on
 * one stream are safe. The buffer keeps the last call's partials; nothing in
 * it needs to start at zero.
 */
#define PA_NOALLOC_WORKSPACE_BYTES (64u * 1024u * 1024u)
pa_status_t pa_decode_partitioned_noalloc(void* out, pa_dtype_t out_dtype, const void* query,
                                          const void* key_cache, const void* value_cache,
                                          pa_dtype_t kv_dtype, const int32_t* block_tables,
                                          int max_blocks_per_seq, const int32_t* context_lens,
                                          int num_seqs, int num_q_heads, int num_kv_heads,
                                          int head_size, int block_size, int64_t num_blocks,
                                          float scale, int max_context_len, int partition_size,
                                          void* stream);

/*
 * Workspace bytes pa_decode_balanced and pa_decode_step need: with
 * G = num_q_heads / num_kv_heads and W = 1024 (the most workgroups a call
 * launches), 256-byte-aligned arrays of W 16-byte descriptors, then float32
 * part_max [2W][G], part_sum [2W][G] and part_out [2W][G][head_size]. It does
 * not depend on the batch. Returns 0 for arguments out of range.
 */
size_t pa_decode_balanced_workspace_size(int num_q_heads, int num_kv_heads, int head_size);

/*
 * pa_decode_balanced -- paged decode attention with the work split evenly by
 * bytes read, not by sequence.
 *
 * Same inputs and result as pa_decode (the attention of each sequence's query
 * over all L = context_lens[s] tokens of its context, read through its block
 * table: "The idea vLLM started from: pages" on "What vLLM Is and Why It
 * Exists"). Contexts of very different lengths share one step (the pages'
 * traffic is mostly short requests and a few long ones, "The problem a naive
 * server has"), so the 16-token blocks of every (sequence, KV head) row are
 * laid end to end and cut into equal contiguous ranges: one per resident
 * workgroup, and within it one per wave. A row split between ranges is
 * finished with the log-sum-exp combination of its pieces (as
 * pa_decode_partitioned combines partitions) in a fixed order, by the
 * workgroup itself when the split is inside it, else by a second small
 * kernel. The result equals pa_decode up to fp32 rounding order; it depends
 * only on the context lengths and the number of compute units, never on
 * block placement, and repeats bit for bit.
 *
 *   workspace  device scratch of at least pa_decode_balanced_workspace_size()
 *              bytes, 256-byte aligned; its contents before the call do not
 *              matter and are unspecified after it. Two calls sharing a
 *              workspace must not overlap in time.
 *   num_seqs   0 .. 4096 (PA_EUNSUPPORTED above), and
 *              num_seqs * num_kv_heads * max_blocks_per_seq < 2^31.
 * Other arguments, checks, errors and the NaN rows of unreadable contexts
 * (longer than 16 * max_blocks_per_seq tokens, or reaching a block id outside
 * [0, NB)) are those of pa_decode.
 */
pa_status_t pa_decode_balanced(void* out, pa_dtype_t out_dtype, const void* query,
                               const void* key_cache, const void* value_cache, pa_dtype_t kv_dtype,
                               const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* context_lens, int num_seqs, int num_q_heads,
                               int num_kv_heads, int head_size, int block_size, int64_t num_blocks,
                               float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_step -- one decode step in one call: write each sequence's new
 * token into the cache and attend over the context that includes it.
 *
 * Each request keeps the key/value vectors of every token it produced ("The
 * problem a naive server has", point 3, on "What vLLM Is and Why It Exists").
 * For every sequence s with L = context_lens[s] >= 1 (L counts the new
 * token), key[s][h][:] and value[s][h][:] are written into row (L - 1) % 16 of
 * physical block block_tables[s][(L - 1) / 16] of both pools, for every KV
 * head h -- exactly what pa_reshape_and_cache does with slot =
 * block_tables[s][(L - 1) / 16] * 16 + (L - 1) % 16 -- and out is the
 * attention of pa_decode_balanced over the L tokens, the new one included
 * (taken from key/value directly, so the result does not depend on when the
 * write lands). A sequence with L = 0, an unreadable context, or a table entry
 * for position L - 1 outside [0, NB) writes nothing.
 *
 *   key, value  [S][Hkv][D] of kv_dtype (device), 16-byte aligned.
 *   key_cache, value_cache  updated in place (one slot per sequence).
 * The block holding position L - 1 must not be shared with another sequence
 * in the call (copy-on-write first: pa_copy_blocks). Other arguments, checks
 * and errors as pa_decode_balanced; key or value null with num_seqs > 0 is
 * PA_EINVAL.
 */
pa_status_t pa_decode_step(void* out, pa_dtype_t out_dtype, const void* query, const void* key,
                           const void* value, void* key_cache, void* value_cache,
                           pa_dtype_t kv_dtype, const int32_t* block_tables, int max_blocks_per_seq,
                           const int32_t* context_lens, int num_seqs, int num_q_heads,
                           int num_kv_heads, int head_size, int block_size, int64_t num_blocks,
                           float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_partitioned_step -- the same decode step (write each sequence's
 * new token into the cache and attend over the context that includes it) on
 * the partitioned schedule of pa_decode_partitioned.
 *
 * The write is that of pa_decode_step: key[s][h][:] and value[s][h][:] go to
 * row (L - 1) % 16 of block block_tables[s][(L - 1) / 16] of both pools for
 * every sequence with L = context_lens[s] >= 1 whose context is readable and
 * whose entry for position L - 1 lies in [0, NB). out is the attention of
 * pa_decode_partitioned over the L tokens, the new one taken from key/value
 * directly (by the partition that holds position L - 1; the pools are read
 * only below it). Same result as pa_reshape_and_cache followed by
 * pa_decode_partitioned up to fp32 rounding order.
 *
 *   key, value  [S][Hkv][D] of kv_dtype (device), 16-byte aligned.
 *   key_cache, value_cache  updated in place (one slot per sequence).
 * The block holding position L - 1 must not be shared with another sequence
 * in the call. Workspace, partition size and every other argument, check and
 * error as pa_decode_partitioned; key or value null with num_seqs > 0 is
 * PA_EINVAL.
 */
pa_status_t pa_decode_partitioned_step(void* out, pa_dtype_t out_dtype, const void* query,
                                       const void* key, const void* value, void* key_cache,
                                       void* value_cache, pa_dtype_t kv_dtype,
                                       const int32_t* block_tables, int max_blocks_per_seq,
                                       const int32_t* context_lens, int num_seqs,
                                       int num_q_heads, int num_kv_heads, int head_size,
                                       int block_size, int64_t num_blocks, float scale,
                                       int max_context_len, int partition_size, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * Workspace bytes pa_decode_cascade needs. With
 *   NPs = max(1, ceil(max(max_context_len - 16 * num_prefix_blocks, 0) / partition_size))
 *   NC  = ceil(num_prefix_blocks / 32),  NP = NPs + NC,  R = S * Hq * NP,
 * the layout and size formula are those of the partitioned workspace:
 *     2 * round_up(4 R, 256) + round_up(4 R D, 256).
 * Returns 0 when an argument is out of range.
 */
size_t pa_decode_cascade_workspace_size(int num_seqs, int num_q_heads, int head_size,
                                        int max_context_len, int partition_size,
                                        int num_prefix_blocks);

/*
 * pa_decode_cascade -- decode attention over a shared prefix plus per-sequence
 * suffixes.
 *
 * Two requests with a common prefix can map the same physical blocks ("Idea
 * 1: PagedAttention" on the day-9 post, "Why this wins"). When the first
 * num_prefix_blocks entries of EVERY block table are the same block ids, the
 * prefix keys and values are the same for every sequence, so the prefix part
 * of the attention is one dense product per KV head over all S * G query rows
 * (G = Hq / Hkv). This call computes:
 *   1. the prefix, in chunks of 32 or 64 blocks, for all query rows at once (K and V
 *      read once per KV head, not once per sequence);
 *   2. each sequence's suffix, tokens [16 * num_prefix_blocks, L), through
 *      block-table entries num_prefix_blocks .. MB - 1, in partitions of
 *      partition_size tokens (as pa_decode_partitioned);
 *   3. the log-sum-exp combination of the prefix chunks and suffix partitions
 *      (the same formula as pa_decode_partitioned).
 * Steps 1 and 2 write disjoint workspace slots; when the suffixes run on the
 * persistent schedule they share one launch (some workgroups take prefix
 * tiles of 64 blocks, the rest decode suffixes), otherwise they are two
 * launches (prefix chunks of 32 blocks). Both give the same attention, up to
 * fp32 rounding order.
 * The result equals pa_decode on the same inputs, up to fp32 rounding order:
 * the same softmax attention of each query over all L tokens of its context.
 * (The pages name the sharing but give no kernel for it; this split is the
 * standard log-sum-exp decomposition of softmax over disjoint token sets.)
 *
 *   kv_dtype           PA_BF16 only (PA_EUNSUPPORTED otherwise); out_dtype
 *                      PA_F32 or PA_BF16.
 *   num_prefix_blocks  1 <= num_prefix_blocks <= MB. The prefix ids are read
 *                      from row 0 of block_tables; the caller guarantees that
 *                      every other row starts with the same ids (the call
 *                      does not compare them). Every context must hold the
 *                      whole prefix: L < 16 * num_prefix_blocks gives a NaN
 *                      row, as does a prefix id outside [0, NB) (for every
 *                      sequence) or a suffix id outside [0, NB).
 *   max_context_len    an upper bound on every context_lens[s]; it sizes the
 *                      suffix partitions. A context whose suffix (tokens past
 *                      the prefix) is longer than NPs * partition_size
 *                      tokens (NPs below) gives a NaN row.
 *   partition_size     suffix tokens per partition, a positive multiple of 16.
 *   num_blocks         NB >= 1 (PA_EINVAL for an empty pool).
 *   workspace          device scratch of at least
 *                      pa_decode_cascade_workspace_size(...) bytes, 256-byte
 *                      aligned, float32 part_max [S][Hq][NP], part_sum
 *                      [S][Hq][NP], part_out [S][Hq][NP][D]: slots
 *                      0 .. NPs - 1 of a row hold suffix partitions, slots
 *                      NPs .. NP - 1 the prefix chunks. Its contents before
 *                      the call do not matter; after it they are unspecified.
 *   num_seqs = 0 is valid and enqueues nothing. Other arguments and errors
 *   are those of pa_decode_partitioned.
 */
pa_status_t pa_decode_cascade(void* out, pa_dtype_t out_dtype, const void* query,
                              const void* key_cache, const void* value_cache, pa_dtype_t kv_dtype,
                              const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* context_lens, int num_seqs, int num_q_heads,
                              int num_kv_heads, int head_size, int block_size, int64_t num_blocks,
                              float scale, int num_prefix_blocks, int max_context_len,
                              int partition_size, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * pa_prefill -- multi-token queries over the paged cache (a prompt, or a
 * chunk of one, whose K and V were already written with
 * pa_reshape_and_cache).
 *
 * "Problem 1" on "vLLM Solved the Wrong Bottleneck" follows a prompt and then
 * each generated token, every one of which needs the keys and values of all
 * tokens before it; the paged cache keeps them in blocks reached through the
 * block table ("The idea vLLM started from: pages" on "What vLLM Is and Why It
 * Exists"). Reading (no formula on the pages): sequence s brings
 * q_s = query_start[s + 1] - query_start[s] query rows, the last q_s tokens
 * of its context of L = context_lens[s] tokens. Row i (query row
 * query_start[s] + i) sits at position pos = L - q_s + i; for each query
 * head h (KV head k = h / G):
 *     out[row][h][:] = sum_{t <= pos} softmax_t(scale * q[row][h] . K_t) V_t
 * with K_t, V_t read through the table as in pa_decode. q_s = 1 is a decode
 * step; q_s = L is a whole prompt.
 *
 *   out              [T][Hq][D], T = query_start[S]; PA_F32 or PA_BF16.
 *   query            [T][Hq][D], bf16 (the kv_dtype).
 *   key_cache,
 *   value_cache      [NB][Hkv][16][D], bf16 (PA_EUNSUPPORTED otherwise).
 *   query_start      int32 [S + 1], device: 0 = query_start[0] <=
 *                    query_start[1] <= ... <= T; rows of sequence s are
 *                    query_start[s] .. query_start[s + 1] - 1.
 *   num_query_rows   T, the rows of query and out (>= 0; 0 enqueues nothing).
 *                    A sequence whose rows do not lie inside [0, T) is
 *                    skipped (nothing read or written for it).
 *   max_query_len    an upper bound on every q_s, known on the host; it sizes
 *                    the grid. Of a longer q_s only the first max_query_len
 *                    rows are computed (at their positions L - q_s + i); the
 *                    rest are not written.
 *   Other arguments, alignment and status codes as pa_decode; max_query_len
 *   < 0 or num_query_rows < 0 is PA_EINVAL; num_seqs = 0, max_query_len = 0
 *   or num_query_rows = 0 enqueues nothing.
 *   workspace        device scratch of at least pa_prefill_workspace_size()
 *                    bytes, 256-byte aligned (null or smaller:
 *                    PA_EWORKSPACE); its contents before the call do not
 *                    matter. The call first orders its work there (the
 *                    longest contexts' row tiles first); two calls sharing a
 *                    workspace must not overlap in time. The order never
 *                    changes a result: every row is computed the same way.
 *   Device-side: a sequence with q_s > L, a context longer than its table
 *   (L > 16 MB) or an empty pool gets NaN rows; a table id outside [0, NB)
 *   within the context gives NaN rows for that sequence (no load leaves the
 *   pool). Nothing is allocated; the call is asynchronous on `stream`.
 */
size_t pa_prefill_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads,
                                 int max_query_len);
pa_status_t pa_prefill(void* out, pa_dtype_t out_dtype, const void* query,
                       const void* key_cache, const void* value_cache, pa_dtype_t kv_dtype,
                       const int32_t* block_tables, int max_blocks_per_seq,
                       const int32_t* context_lens, const int32_t* query_start,
                       int64_t num_query_rows, int num_seqs, int num_q_heads, int num_kv_heads,
                       int head_size, int block_size, int64_t num_blocks, float scale,
                       int max_query_len, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Block manager -- host-side owner of the pool's blocks and of every
 * sequence's block table (the producer of the block_tables, slot_mapping and
 * copy-on-write block_mapping arguments above).
 *
 * "Idea 1: PagedAttention" on the day-9 post: the cache is split into
 * fixed-size blocks, a block table maps a request's logical blocks to
 * physical ones, requests with a common prefix share physical blocks, and a
 * shared block that must diverge is copied alone ("Why this wins"). "The idea
 * vLLM started from: pages" on "What vLLM Is and Why It Exists": blocks are
 * handed out on demand; "preemption" takes a request's blocks away to feed
 * another. Readings where the pages are silent:
 *   - free blocks form a stack, initially with block 0 on top (a fresh pool
 *     hands out 0, 1, 2, ...); a released block goes on top;
 *   - releasing a table walks it from its first entry to its last; a block is
 *     free again when no table holds it;
 *   - adding a sequence takes all of its blocks or none (PA_ENOSPACE);
 *   - appending the token at position L takes a new block when L is a
 *     multiple of block_size; otherwise, if the last block is shared, it is
 *     replaced by a fresh block and (old, new) is reported: the caller copies
 *     block old onto block new (pa_copy_blocks) before writing the token;
 *   - slot of position t = table[t / block_size] * block_size + t % block_size.
 * Preempting a sequence is pa_bm_free_sequence; choosing the victim is the
 * caller's. Host memory only (no GPU call). One manager must not be used from
 * two threads at once; different managers are independent.
 */
typedef struct pa_block_manager pa_block_manager;

/* A manager of num_blocks (0 .. INT32_MAX) blocks of block_size tokens; NULL
 * for bad arguments or when host memory runs out. */
pa_block_manager* pa_bm_create(int64_t num_blocks, int block_size);
void pa_bm_destroy(pa_block_manager* bm);

/* A new sequence seq_id of num_tokens >= 0 tokens: ceil(num_tokens /
 * block_size) blocks, and slots_out[t] (host array of num_tokens) = the slot
 * of token t. PA_EINVAL for an id in use or a negative count; PA_ENOSPACE
 * (nothing changed) when too few blocks are free. */
pa_status_t pa_bm_add_sequence(pa_block_manager* bm, int64_t seq_id, int num_tokens,
                               int64_t* slots_out);

/* Room for one more token of seq_id: *slot_out = its slot; cow_out[0..1] =
 * (source, destination) block of a copy-on-write the caller must perform
 * first, or (-1, -1). PA_EINVAL for an unknown id; PA_ENOSPACE (nothing
 * changed) when a block is needed and none is free. */
pa_status_t pa_bm_append_token(pa_block_manager* bm, int64_t seq_id, int64_t* slot_out,
                               int64_t* cow_out);

/* child_id (a new id) gets parent_id's table and length; every block of it is
 * now shared. PA_EINVAL for an unknown parent or an id in use. */
pa_status_t pa_bm_fork(pa_block_manager* bm, int64_t parent_id, int64_t child_id);

/* Releases seq_id's table (also how a sequence is preempted). PA_EINVAL for an
 * unknown id. */
pa_status_t pa_bm_free_sequence(pa_block_manager* bm, int64_t seq_id);

/* Free blocks (-1 for a NULL manager). */
int64_t pa_bm_num_free_blocks(const pa_block_manager* bm);

/* Tokens held by seq_id, or -1 for an unknown id. */
int64_t pa_bm_length(const pa_block_manager* bm, int64_t seq_id);

/* Writes seq_id's block table to table_out[0 .. max_entries) (host), padding
 * past its end with `pad`; returns its number of blocks (which may exceed
 * max_entries), or -1 for an unknown id or bad arguments. */
int64_t pa_bm_block_table(const pa_block_manager* bm, int64_t seq_id, int32_t* table_out,
                          int max_entries, int32_t pad);

/*
 * pa_stream_read -- streaming-read calibration: the HBM read rate this GPU
 * reaches, the practical ceiling of the bandwidth-bound decode kernels.
 *
 * Reads each of the num_words 16-byte words at src once, with the 16-byte
 * nontemporal loads the decode kernels use for K and V, over num_workgroups
 * workgroups of 4 waves, and writes one 16-byte word per wave to sink: the
 * XOR of the words that wave read. The XOR of all 4 * num_workgroups sink
 * words equals the XOR of all words of src, whatever num_workgroups is.
 *
 *   src            device memory, 16-byte aligned, num_words * 16 bytes
 *                  (may be null when num_words = 0).
 *   sink           device memory, 16-byte aligned, 64 * num_workgroups bytes;
 *                  every word is written (zero for a wave that read nothing).
 *   num_workgroups 1 .. 2^20.
 *
 * PA_EINVAL for a negative num_words, num_workgroups out of range, a null or
 * misaligned pointer; PA_EHIP for a launch failure. Nothing is retained.
 */
pa_status_t pa_stream_read(const void* src, int64_t num_words, void* sink, int num_workgroups,
                           void* stream);

/* A static, human-readable name for a status code. */
const char* pa_status_str(pa_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */

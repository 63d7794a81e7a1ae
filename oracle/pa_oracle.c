/*
 * pa_oracle.c -- plain fp64 CPU oracle for paged KV-cache decode attention,
 * multi-token queries over the paged cache, the KV-cache write, the
 * copy-on-write block copy and the swap of blocks between two pools.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the package smoke check and the
 * CPU-baseline leg of the benchmark are the only code that may load this
 * library. It shares no source, header, table or constant with the GPU
 * library, and it is deliberately slow: it follows the definitions below
 * loop by loop, with no blocking, fusion or reordering.
 *
 * What is computed, and where the pages say so:
 *
 *  - KV blocks and the block table. "Idea 1: PagedAttention" (day-9 post,
 *    skandtandon.pages.dev): the KV cache is split into fixed-size blocks,
 *    typically 16 tokens each, and a block table maps a request's logical
 *    blocks to physical blocks. "The idea vLLM started from: pages" ("What
 *    vLLM Is and Why It Exists"): attention reads a request's KV cache from
 *    blocks scattered anywhere in the tensor, following the block table.
 *    "Paged Attention" ("vLLM Solved the Wrong Bottleneck"): each block holds
 *    the key and value vectors of a fixed number of tokens.
 *
 *  - Layout (a reading; the pages give none). Each pool is
 *    [num_blocks][num_kv_heads][block_size][head_size], row-major. Logical
 *    token t of sequence s lives in physical block block_tables[s][t / B] at
 *    row t % B.
 *
 *  - Attention (a reading; the pages print no formula). The single new query
 *    of each sequence attends over all L_s tokens of its context with
 *    standard scaled dot-product softmax attention. Query head h reads KV
 *    head h / (Hq / Hkv): consecutive query heads share a KV head.
 *
 *        l_t   = scale * sum_d q[h][d] * K_t[d]
 *        w_t   = exp(l_t - max_u l_u) / sum_u exp(l_u - max_u l_u)
 *        out_h = sum_t w_t * V_t
 *
 *    A context length of 0 gives a zero row.
 *
 *  - Split-context form (a reading). The context is cut into partitions of
 *    partition_size tokens; each partition p yields its own maximum m_p, sum
 *    s_p = sum exp(l_t - m_p) and normalised output o_p, and the partitions
 *    are combined with log-sum-exp weights s_p * exp(m_p - M), M = max m_p.
 *    In exact arithmetic this equals the single-pass result.
 *
 *  - Multi-token queries (a reading). "Problem 1" on "vLLM Solved the Wrong
 *    Bottleneck" walks through a 1000-token prompt followed by generated
 *    tokens, each of which attends to all tokens before it. Sequence s brings
 *    q_s new tokens, the last q_s of its L_s-token context (already written
 *    to the cache); its query token i sits at position pos = L_s - q_s + i
 *    and attends, causally, to tokens 0 .. pos with the same softmax
 *    attention. q_s = 1 is the decode above.
 *
 *  - KV-cache write (a reading). Each new token i with slot_mapping[i] >= 0
 *    is copied byte for byte into row slot % B of block slot / B, for every
 *    KV head. A negative slot marks a padding token and is skipped. Two
 *    tokens naming the same slot is an input error.
 *
 * All floating-point work is fp64 on values already converted exactly from
 * the stored inputs.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum {
    ORACLE_OK = 0,
    ORACLE_BAD_ARG = -1,    /* a count, size or pointer is invalid               */
    ORACLE_BAD_BLOCK = -2,  /* a table entry inside the context is outside pool  */
    ORACLE_BAD_LEN = -3,    /* a context length is negative or beyond the table  */
    ORACLE_BAD_SLOT = -4,   /* a slot lies past the end of the pool              */
    ORACLE_DUP_SLOT = -5,   /* two tokens write the same slot                    */
    ORACLE_NOMEM = -6,
    ORACLE_BAD_PAIR = -7    /* a block copy whose order would matter, or past pool */
};

/* ------------------------------------------------------------------------ */
/* KV-cache write                                                           */
/* ------------------------------------------------------------------------ */

static int cmp_i64(const void* a, const void* b)
{
    int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
    return (x > y) - (x < y);
}

int oracle_reshape_and_cache(const uint8_t* key, const uint8_t* value,
                             uint8_t* key_cache, uint8_t* value_cache,
                             const int64_t* slot_mapping, int64_t num_tokens,
                             int num_kv_heads, int head_size, int block_size,
                             int64_t num_blocks, int elem_bytes)
{
    if (num_tokens < 0 || num_kv_heads <= 0 || head_size <= 0 || block_size <= 0 ||
        num_blocks < 0 || elem_bytes <= 0)
        return ORACLE_BAD_ARG;
    if (num_tokens == 0)
        return ORACLE_OK;

    /* Check every slot before writing anything. */
    int64_t* sorted = (int64_t*)malloc((size_t)num_tokens * sizeof(int64_t));
    if (!sorted)
        return ORACLE_NOMEM;
    int64_t n_live = 0;
    for (int64_t i = 0; i < num_tokens; ++i) {
        int64_t slot = slot_mapping[i];
        if (slot < 0)
            continue;
        if (slot >= num_blocks * (int64_t)block_size) {
            free(sorted);
            return ORACLE_BAD_SLOT;
        }
        sorted[n_live++] = slot;
    }
    qsort(sorted, (size_t)n_live, sizeof(int64_t), cmp_i64);
    for (int64_t i = 1; i < n_live; ++i) {
        if (sorted[i] == sorted[i - 1]) {
            free(sorted);
            return ORACLE_DUP_SLOT;
        }
    }
    free(sorted);

    const size_t row = (size_t)head_size * (size_t)elem_bytes;   /* one token, one head */
    for (int64_t i = 0; i < num_tokens; ++i) {
        int64_t slot = slot_mapping[i];
        if (slot < 0)
            continue;
        int64_t block = slot / block_size;
        int64_t offset = slot % block_size;
        for (int h = 0; h < num_kv_heads; ++h) {
            size_t dst = (size_t)(((block * num_kv_heads + h) * block_size + offset)) * row;
            size_t src = (size_t)(i * num_kv_heads + h) * row;
            memcpy(key_cache + dst, key + src, row);
            memcpy(value_cache + dst, value + src, row);
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Decode attention                                                         */
/* ------------------------------------------------------------------------ */

static int check_tables(const int32_t* block_tables, const int32_t* context_lens,
                        int num_seqs, int block_size, int max_blocks_per_seq,
                        int64_t num_blocks)
{
    for (int s = 0; s < num_seqs; ++s) {
        int L = context_lens[s];
        if (L < 0 || (int64_t)L > (int64_t)max_blocks_per_seq * block_size)
            return ORACLE_BAD_LEN;
        int nblk = (L + block_size - 1) / block_size;
        for (int j = 0; j < nblk; ++j) {
            int32_t b = block_tables[(int64_t)s * max_blocks_per_seq + j];
            if (b < 0 || (int64_t)b >= num_blocks)
                return ORACLE_BAD_BLOCK;
        }
    }
    return ORACLE_OK;
}

/* Copy the L tokens of KV head `kv` of sequence `s` out of the pool into a
 * contiguous [L][head_size] buffer, following the block table. */
static void gather_head(double* dst, const double* pool, const int32_t* table_row,
                        int L, int kv, int num_kv_heads, int block_size, int head_size)
{
    for (int t = 0; t < L; ++t) {
        int64_t block = table_row[t / block_size];
        int64_t row = (block * num_kv_heads + kv) * block_size + t % block_size;
        memcpy(dst + (size_t)t * head_size, pool + (size_t)row * head_size,
               (size_t)head_size * sizeof(double));
    }
}

/* Scaled logits of one query against tokens [t0, t1) of a gathered head. */
static void logits_range(double* l, const double* qh, const double* K, int t0, int t1,
                         int head_size, double scale)
{
    for (int t = t0; t < t1; ++t) {
        double dot = 0.0;
        for (int d = 0; d < head_size; ++d)
            dot += qh[d] * K[(size_t)t * head_size + d];
        l[t] = scale * dot;
    }
}

int oracle_decode(double* out, const double* query,
                  const double* key_cache, const double* value_cache,
                  const int32_t* block_tables, const int32_t* context_lens,
                  int num_seqs, int num_q_heads, int num_kv_heads, int head_size,
                  int block_size, int max_blocks_per_seq, int64_t num_blocks,
                  double scale, int num_threads)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 ||
        block_size <= 0 || max_blocks_per_seq <= 0 || num_q_heads % num_kv_heads != 0)
        return ORACLE_BAD_ARG;
    int rc = check_tables(block_tables, context_lens, num_seqs, block_size,
                          max_blocks_per_seq, num_blocks);
    if (rc != ORACLE_OK)
        return rc;

    const int group = num_q_heads / num_kv_heads;
    const int64_t pairs = (int64_t)num_seqs * num_kv_heads;
    int failed = 0;
#ifdef _OPENMP
    if (num_threads > 0)
        omp_set_num_threads(num_threads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
    for (int64_t pr = 0; pr < pairs; ++pr) {
        const int s = (int)(pr / num_kv_heads);
        const int kv = (int)(pr % num_kv_heads);
        const int L = context_lens[s];
        if (L == 0) {
            for (int g = 0; g < group; ++g)
                memset(out + ((size_t)s * num_q_heads + kv * group + g) * head_size, 0,
                       (size_t)head_size * sizeof(double));
            continue;
        }
        const int32_t* table_row = block_tables + (int64_t)s * max_blocks_per_seq;
        double* K = (double*)malloc((size_t)L * head_size * sizeof(double));
        double* V = (double*)malloc((size_t)L * head_size * sizeof(double));
        double* l = (double*)malloc((size_t)L * sizeof(double));
        if (!K || !V || !l) {
            free(K); free(V); free(l);
            failed = 1;
            continue;
        }
        gather_head(K, key_cache, table_row, L, kv, num_kv_heads, block_size, head_size);
        gather_head(V, value_cache, table_row, L, kv, num_kv_heads, block_size, head_size);

        for (int g = 0; g < group; ++g) {
            const int h = kv * group + g;
            const double* qh = query + ((size_t)s * num_q_heads + h) * head_size;
            double* o = out + ((size_t)s * num_q_heads + h) * head_size;

            logits_range(l, qh, K, 0, L, head_size, scale);
            double m = -INFINITY;
            for (int t = 0; t < L; ++t)
                if (l[t] > m)
                    m = l[t];
            double z = 0.0;
            for (int t = 0; t < L; ++t) {
                l[t] = exp(l[t] - m);
                z += l[t];
            }
            for (int d = 0; d < head_size; ++d)
                o[d] = 0.0;
            for (int t = 0; t < L; ++t) {
                const double w = l[t] / z;
                for (int d = 0; d < head_size; ++d)
                    o[d] += w * V[(size_t)t * head_size + d];
            }
        }
        free(K); free(V); free(l);
    }
    return failed ? ORACLE_NOMEM : ORACLE_OK;
}

/* Multi-token queries. query and out are [T][num_q_heads][head_size] with
 * T = query_start[num_seqs]; the q_s = query_start[s + 1] - query_start[s]
 * rows of sequence s start at row query_start[s]. Row i of sequence s is the
 * query at context position L_s - q_s + i and attends to tokens 0 .. that
 * position. Requires query_start[0] = 0, non-decreasing, and q_s <= L_s. */
int oracle_prefill(double* out, const double* query,
                   const double* key_cache, const double* value_cache,
                   const int32_t* block_tables, const int32_t* context_lens,
                   const int32_t* query_start,
                   int num_seqs, int num_q_heads, int num_kv_heads, int head_size,
                   int block_size, int max_blocks_per_seq, int64_t num_blocks,
                   double scale, int num_threads)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 ||
        block_size <= 0 || max_blocks_per_seq <= 0 || num_q_heads % num_kv_heads != 0)
        return ORACLE_BAD_ARG;
    if (num_seqs > 0 && query_start[0] != 0)
        return ORACLE_BAD_ARG;
    for (int s = 0; s < num_seqs; ++s) {
        const int nq = query_start[s + 1] - query_start[s];
        if (nq < 0)
            return ORACLE_BAD_ARG;
        if (nq > context_lens[s])
            return ORACLE_BAD_LEN;
    }
    int rc = check_tables(block_tables, context_lens, num_seqs, block_size,
                          max_blocks_per_seq, num_blocks);
    if (rc != ORACLE_OK)
        return rc;

    const int group = num_q_heads / num_kv_heads;
    const int64_t pairs = (int64_t)num_seqs * num_kv_heads;
    int failed = 0;
#ifdef _OPENMP
    if (num_threads > 0)
        omp_set_num_threads(num_threads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
    for (int64_t pr = 0; pr < pairs; ++pr) {
        const int s = (int)(pr / num_kv_heads);
        const int kv = (int)(pr % num_kv_heads);
        const int L = context_lens[s];
        const int nq = query_start[s + 1] - query_start[s];
        if (nq == 0)
            continue;
        const int32_t* table_row = block_tables + (int64_t)s * max_blocks_per_seq;
        double* K = (double*)malloc((size_t)L * head_size * sizeof(double));
        double* V = (double*)malloc((size_t)L * head_size * sizeof(double));
        double* e = (double*)malloc((size_t)L * sizeof(double));
        if (!K || !V || !e) {
            free(K); free(V); free(e);
            failed = 1;
            continue;
        }
        gather_head(K, key_cache, table_row, L, kv, num_kv_heads, block_size, head_size);
        gather_head(V, value_cache, table_row, L, kv, num_kv_heads, block_size, head_size);

        for (int i = 0; i < nq; ++i) {
            const int pos = L - nq + i;            /* the query's own position */
            const int64_t row = (int64_t)query_start[s] + i;
            for (int hh = 0; hh < group; ++hh) {
                const int head = kv * group + hh;
                const double* qh = query + ((size_t)row * num_q_heads + head) * head_size;
                double* o = out + ((size_t)row * num_q_heads + head) * head_size;
                logits_range(e, qh, K, 0, pos + 1, head_size, scale);
                double mx = -INFINITY;
                for (int t = 0; t <= pos; ++t)
                    mx = e[t] > mx ? e[t] : mx;
                double sum = 0.0;
                for (int t = 0; t <= pos; ++t) {
                    e[t] = exp(e[t] - mx);
                    sum += e[t];
                }
                for (int d = 0; d < head_size; ++d)
                    o[d] = 0.0;
                for (int t = 0; t <= pos; ++t)
                    for (int d = 0; d < head_size; ++d)
                        o[d] += e[t] / sum * V[(size_t)t * head_size + d];
            }
        }
        free(K); free(V); free(e);
    }
    return failed ? ORACLE_NOMEM : ORACLE_OK;
}

/* Split-context form. Writes the final output and, when the pointers are not
 * NULL, the per-partition statistics:
 *     part_max[s][h][p], part_sum[s][h][p]    [num_seqs][num_q_heads][num_partitions]
 *     part_out[s][h][p][d]                    normalised partial outputs
 * Partitions past ceil(L / partition_size) get max -inf, sum 0, output 0. */
int oracle_decode_partitioned(double* out, double* part_max, double* part_sum,
                              double* part_out, const double* query,
                              const double* key_cache, const double* value_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int num_seqs, int num_q_heads, int num_kv_heads,
                              int head_size, int block_size, int max_blocks_per_seq,
                              int64_t num_blocks, double scale, int partition_size,
                              int num_partitions, int num_threads)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 ||
        block_size <= 0 || max_blocks_per_seq <= 0 || num_q_heads % num_kv_heads != 0 ||
        partition_size <= 0 || num_partitions <= 0)
        return ORACLE_BAD_ARG;
    int rc = check_tables(block_tables, context_lens, num_seqs, block_size,
                          max_blocks_per_seq, num_blocks);
    if (rc != ORACLE_OK)
        return rc;
    for (int s = 0; s < num_seqs; ++s)
        if ((int64_t)context_lens[s] > (int64_t)num_partitions * partition_size)
            return ORACLE_BAD_LEN;

    const int group = num_q_heads / num_kv_heads;
    const int64_t pairs = (int64_t)num_seqs * num_kv_heads;
    int failed = 0;
#ifdef _OPENMP
    if (num_threads > 0)
        omp_set_num_threads(num_threads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
    for (int64_t pr = 0; pr < pairs; ++pr) {
        const int s = (int)(pr / num_kv_heads);
        const int kv = (int)(pr % num_kv_heads);
        const int L = context_lens[s];
        const int np_s = (L + partition_size - 1) / partition_size;
        const int32_t* table_row = block_tables + (int64_t)s * max_blocks_per_seq;
        double* K = (double*)malloc(((size_t)L + 1) * head_size * sizeof(double));
        double* V = (double*)malloc(((size_t)L + 1) * head_size * sizeof(double));
        double* l = (double*)malloc(((size_t)L + 1) * sizeof(double));
        double* mp = (double*)malloc((size_t)num_partitions * sizeof(double));
        double* sp = (double*)malloc((size_t)num_partitions * sizeof(double));
        double* op = (double*)malloc((size_t)num_partitions * head_size * sizeof(double));
        if (!K || !V || !l || !mp || !sp || !op) {
            free(K); free(V); free(l); free(mp); free(sp); free(op);
            failed = 1;
            continue;
        }
        gather_head(K, key_cache, table_row, L, kv, num_kv_heads, block_size, head_size);
        gather_head(V, value_cache, table_row, L, kv, num_kv_heads, block_size, head_size);

        for (int g = 0; g < group; ++g) {
            const int h = kv * group + g;
            const double* qh = query + ((size_t)s * num_q_heads + h) * head_size;
            double* o = out + ((size_t)s * num_q_heads + h) * head_size;

            /* Each partition on its own. */
            for (int p = 0; p < num_partitions; ++p) {
                double* opp = op + (size_t)p * head_size;
                for (int d = 0; d < head_size; ++d)
                    opp[d] = 0.0;
                mp[p] = -INFINITY;
                sp[p] = 0.0;
                if (p >= np_s)
                    continue;
                const int t0 = p * partition_size;
                const int t1 = (t0 + partition_size < L) ? t0 + partition_size : L;
                logits_range(l, qh, K, t0, t1, head_size, scale);
                for (int t = t0; t < t1; ++t)
                    if (l[t] > mp[p])
                        mp[p] = l[t];
                for (int t = t0; t < t1; ++t) {
                    l[t] = exp(l[t] - mp[p]);
                    sp[p] += l[t];
                }
                for (int t = t0; t < t1; ++t) {
                    const double w = l[t] / sp[p];
                    for (int d = 0; d < head_size; ++d)
                        opp[d] += w * V[(size_t)t * head_size + d];
                }
            }

            /* Log-sum-exp combination of the partitions. */
            double M = -INFINITY;
            for (int p = 0; p < np_s; ++p)
                if (mp[p] > M)
                    M = mp[p];
            double wsum = 0.0;
            for (int d = 0; d < head_size; ++d)
                o[d] = 0.0;
            for (int p = 0; p < np_s; ++p) {
                const double w = sp[p] * exp(mp[p] - M);
                wsum += w;
                for (int d = 0; d < head_size; ++d)
                    o[d] += w * op[(size_t)p * head_size + d];
            }
            if (np_s > 0)
                for (int d = 0; d < head_size; ++d)
                    o[d] /= wsum;

            if (part_max && part_sum && part_out) {
                for (int p = 0; p < num_partitions; ++p) {
                    const size_t idx = ((size_t)s * num_q_heads + h) * num_partitions + p;
                    part_max[idx] = mp[p];
                    part_sum[idx] = sp[p];
                    memcpy(part_out + idx * head_size, op + (size_t)p * head_size,
                           (size_t)head_size * sizeof(double));
                }
            }
        }
        free(K); free(V); free(l); free(mp); free(sp); free(op);
    }
    return failed ? ORACLE_NOMEM : ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Block copy (copy-on-write)                                               */
/* ------------------------------------------------------------------------ */

/*
 * Copy-on-write ("Idea 1: PagedAttention", day-9 post, "Why this wins": when a
 * shared block has to diverge, only the changed block is copied, not the
 * whole cache). Each pair (src, dst) of block_mapping copies physical block
 * src of both pools -- every KV head, every row, block_bytes bytes per pool --
 * onto block dst, byte for byte. A pair with a negative id is skipped. A
 * destination must not repeat and must not be any pair's source, so that the
 * result cannot depend on the order of the copies; ids past the pool are
 * errors too. Nothing is written when a check fails.
 */
int oracle_copy_blocks(uint8_t* key_cache, uint8_t* value_cache, const int64_t* block_mapping,
                       int64_t num_pairs, int64_t block_bytes, int64_t num_blocks)
{
    if (num_pairs < 0 || block_bytes <= 0 || num_blocks < 0)
        return ORACLE_BAD_ARG;
    for (int64_t i = 0; i < num_pairs; ++i) {
        const int64_t src = block_mapping[2 * i], dst = block_mapping[2 * i + 1];
        if (src < 0 || dst < 0)
            continue;
        if (src >= num_blocks || dst >= num_blocks)
            return ORACLE_BAD_PAIR;
        for (int64_t j = 0; j < num_pairs; ++j) {
            const int64_t s2 = block_mapping[2 * j], d2 = block_mapping[2 * j + 1];
            if (s2 < 0 || d2 < 0)
                continue;
            if (dst == s2 || (j != i && dst == d2))
                return ORACLE_BAD_PAIR;
        }
    }
    for (int64_t i = 0; i < num_pairs; ++i) {
        const int64_t src = block_mapping[2 * i], dst = block_mapping[2 * i + 1];
        if (src < 0 || dst < 0)
            continue;
        memcpy(key_cache + dst * block_bytes, key_cache + src * block_bytes, (size_t)block_bytes);
        memcpy(value_cache + dst * block_bytes, value_cache + src * block_bytes, (size_t)block_bytes);
    }
    return ORACLE_OK;
}

/*
 * Swap ("Why read its source at all" on "What vLLM Is and Why It Exists":
 * preemption takes a request's blocks away to feed another; "Idea 1:
 * PagedAttention", day-9 post: the cache lives in fixed-size blocks). A
 * reading: a preempted request's blocks are moved out of the GPU pools into a
 * second pair of pools (host memory) and later back, each block whole --
 * every KV head, every row -- byte for byte. Each pair (src, dst) of
 * block_mapping copies block src of the source pools onto block dst of the
 * destination pools. A pair with a negative id is skipped; an id past its
 * pool, or a destination named twice (the result would depend on the order),
 * is an error and nothing is written. Source and destination pools are
 * different memory.
 */
int oracle_swap_blocks(const uint8_t* src_key, const uint8_t* src_value, int64_t src_num_blocks,
                       uint8_t* dst_key, uint8_t* dst_value, int64_t dst_num_blocks,
                       const int64_t* block_mapping, int64_t num_pairs, int64_t block_bytes)
{
    if (num_pairs < 0 || block_bytes <= 0 || src_num_blocks < 0 || dst_num_blocks < 0)
        return ORACLE_BAD_ARG;
    for (int64_t i = 0; i < num_pairs; ++i) {
        const int64_t src = block_mapping[2 * i], dst = block_mapping[2 * i + 1];
        if (src < 0 || dst < 0)
            continue;
        if (src >= src_num_blocks || dst >= dst_num_blocks)
            return ORACLE_BAD_PAIR;
        for (int64_t j = i + 1; j < num_pairs; ++j)
            if (block_mapping[2 * j] >= 0 && block_mapping[2 * j + 1] == dst)
                return ORACLE_BAD_PAIR;
    }
    for (int64_t i = 0; i < num_pairs; ++i) {
        const int64_t src = block_mapping[2 * i], dst = block_mapping[2 * i + 1];
        if (src < 0 || dst < 0)
            continue;
        memcpy(dst_key + dst * block_bytes, src_key + src * block_bytes, (size_t)block_bytes);
        memcpy(dst_value + dst * block_bytes, src_value + src * block_bytes, (size_t)block_bytes);
    }
    return ORACLE_OK;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

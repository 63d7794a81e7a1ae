// pa_decode.hip -- paged decode attention kernel for gfx950 (CDNA4).
//
// What is computed: for each sequence, its one new query token attends over
// a KV cache held in 16-token blocks scattered through a shared pool and
// reached through the sequence's block table ("Idea 1: PagedAttention" on
// the day-9 post of skandtandon.pages.dev; "The idea vLLM started from:
// pages" on "What vLLM Is and Why It Exists"). The attention is standard
// scaled dot-product softmax attention (the pages print no formula).
//
// Work decomposition. A work item is one context partition of one KV head
// of one sequence; the single-pass entry point is the case of one partition
// that spans the whole table. Every query head of the group that shares the
// KV head is handled by the same wave, so each K/V byte is read from HBM once
// per step. The partitioned entry point runs a persistent schedule: only as
// many workgroups as the GPU keeps resident, whose waves take every V-th item
// (V = the grid's waves) of the items that exist, numbered through a prefix
// sum of the sequences' partition counts built from context_lens in LDS; a
// wave streams its item's blocks alone, one block per round. The single pass,
// and batches whose context lengths do not fit a workgroup's LDS, use one
// workgroup per item instead, its waves taking the item's blocks in turns and
// merging their (max, sum, output) through LDS in a fixed order.
//
// The per-round work of a wave (table resolve, K/V streaming, Q^T K on MFMA,
// online softmax, P.V) is in pa_decode_core.h.
//
// Split contexts. A sequence with a single partition writes its output row
// directly. Otherwise each partition writes its (max, sum, normalised
// output) to the workspace and a second, small kernel combines the
// partitions of each (sequence, KV head) with log-sum-exp weights, in
// partition order. Every reduction runs in an order fixed by logical token
// positions, so results never depend on where the blocks sit in the pool.
#include <algorithm>

#include "pa_cascade_tile.h"
#include "pa_decode_core.h"

namespace pa {
namespace {

using namespace core;

// Writes the output rows of the head group of KV head `kvh` of sequence `s`
// when its context has nothing to read: zeros for an empty context, NaN for
// an unreadable one (by the workgroup, or with SOLO by the calling wave).
template <typename OUT, bool SOLO>
__device__ __forceinline__ void fill_rows(const DecodeParams& p, int kvh, int s, int D, float v) {
    const int G = p.group;
    const int step = SOLO ? kWave : static_cast<int>(blockDim.x);
    for (int idx = SOLO ? (threadIdx.x & (kWave - 1)) : threadIdx.x; idx < G * D; idx += step) {
        const int h = idx / D, d = idx - (idx / D) * D;
        store_out<OUT>(p.out, ((int64_t)s * p.num_q_heads + kvh * G + h) * D + d, v);
    }
}

// Blocks [pb0, pb1) of the context of KV head `kvh` of sequence `s` (L > 0
// tokens, readable), computed by the whole workgroup, or with SOLO by the
// calling wave alone (its own LDS slices, no workgroup barrier; the other
// waves of the workgroup work on other ranges meanwhile). With `direct` the range
// is the whole context and the output row is written; otherwise the range's
// (max, sum, normalised output) go to partial slot `slot` of the workspace.
// With WRITE, the range that holds the context's last token (its new one)
// streams only the tokens before it from the pool; wave 0 (or the SOLO wave)
// takes the new token's K and V from p.new_key / p.new_value, attends to it and stores it
// in its slot, so the attention never reads the slot being written. All
// arguments are wave-uniform.
template <typename KV, int D, int GMAX, typename OUT, bool WRITE, bool SOLO>
__device__ __forceinline__ void process_range(const DecodeParams& p, float* smem, int kvh, int s,
                                              int L, int pb0, int pb1, int slot, bool direct) {
    using Gm = Geometry<KV, D>;
    constexpr int CH = Gm::kCh, EPC = Gm::kEpc, ROW = Gm::kRow;
    constexpr int BPW = decode_bpw(KV::kBytes, D, GMAX);
    constexpr int GP = decode_pstride(GMAX);

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nwl = blockDim.x / kWave;                         // waves in the LDS layout
    const int nw = SOLO ? 1 : nwl;                              // waves sharing this range
    const int w0 = SOLO ? wave : 0;                             // the first of them
    const bool lead = SOLO || wave == 0;                        // takes the new token
    const int per_round = nw * BPW;
    const int lane = threadIdx.x & (kWave - 1);
    const bool with_new = WRITE && pb1 * kBlockSize >= L;      // the range holds token L - 1
    const int L_pool = with_new ? L - 1 : L;
    const int pb1_pool = min(pb1, (L_pool + kBlockSize - 1) / kBlockSize);
    const int rounds = (pb1_pool - pb0 + per_round - 1) / per_round;
    u32x4 qa[Gm::kNq];
    load_query<KV, D>(p, kvh, s, qa);
    NewToken<KV, D> tok;
    if constexpr (WRITE) {
        if (with_new && lead) {
            const int64_t src = ((int64_t)s * p.num_kv_heads + kvh) * ROW;
            tok = load_new_token<KV, D>(static_cast<const char*>(p.new_key) + src,
                                        static_cast<const char*>(p.new_value) + src);
        }
    }
    WaveAcc<KV, D, GMAX> acc;
    acc.reset();
    if (rounds > 0)
        accumulate_blocks<KV, D, GMAX>(p, smem + wave * (BPW * kBlockSize * GP), qa, kvh, s, L_pool,
                                       pb1_pool, pb0 + (wave - w0) * BPW, per_round, rounds, acc);
    if constexpr (WRITE) {
        if (with_new && lead) {
            accumulate_token<KV, D, GMAX>(p, qa, tok, acc);
            store_new_token<KV, D>(p, tok, s, kvh, L, p.skip_blocks);
        }
    }

    const int Hq = p.num_q_heads, G = p.group;
    const int g = lane >> 4;       // MFMA lane group: output rows 4g..4g+3
    const int r16 = lane & 15;
    const int vchunk = lane % CH;  // V layout: chunk within the row
    const int vrow = lane / CH;    //           first token row

    // Wave totals: sums over the 16 token columns, outputs over the token rows.
    float srow[4];
    wave_totals<KV, D, GMAX>(acc, srow);
    float (&m)[4] = acc.m;
    float (&o)[GMAX][EPC] = acc.o;

    float* red_m = smem + nwl * (BPW * kBlockSize * GP);
    float* red_s = red_m + nwl * GP;
    float* red_o = red_s + nwl * GP;
    if (r16 == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int h = 4 * g + j;
            if (h < GMAX) {
                red_m[wave * GP + h] = m[j];
                red_s[wave * GP + h] = srow[j];
            }
        }
    }
    if (vrow == 0) {
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
            float* dst = red_o + (wave * GMAX + h) * D + vchunk * EPC;
#pragma unroll
            for (int e = 0; e < EPC; e += 4)
                *reinterpret_cast<f32x4*>(dst + e) = f32x4{o[h][e], o[h][e + 1], o[h][e + 2], o[h][e + 3]};
        }
    }
    if constexpr (SOLO)
        wave_lds_sync();
    else
        __syncthreads();

    // Merge the waves in a fixed order (a SOLO wave: its own totals, with
    // weight exp2(0) = 1).
    const bool split = !direct;
    const int step = SOLO ? kWave : static_cast<int>(blockDim.x);
    for (int idx = SOLO ? lane : static_cast<int>(threadIdx.x); idx < G * D; idx += step) {
        const int h = idx / D;
        const int d = idx - h * D;
        float M = -INFINITY;
        for (int w = w0; w < w0 + nw; ++w)
            M = fmaxf(M, red_m[w * GP + h]);
        float S = 0.0f, od = 0.0f;
        for (int w = w0; w < w0 + nw; ++w) {
            const float f = __builtin_amdgcn_exp2f(red_m[w * GP + h] - M);
            S = fmaf(red_s[w * GP + h], f, S);
            od = fmaf(red_o[(w * GMAX + h) * D + d], f, od);
        }
        const int64_t row = (int64_t)s * Hq + (int64_t)kvh * G + h;
        if (!split) {
            store_out<OUT>(p.out, row * D + d, od / S);
        } else {
            const int64_t pi = row * p.part_stride + slot;
            p.part_out[pi * D + d] = od / S;
            if (d == 0) {
                p.part_max[pi] = M * kLn2;
                p.part_sum[pi] = S;
            }
        }
    }
}

// Blocks a context spans, as the schedule counts them: a context with nothing
// to read counts one block (its item writes the zero or NaN row).
__device__ __forceinline__ int schedule_blocks(int L, const DecodeParams& p) {
    if (L == 0 || context_unreadable(L, p.table_blocks, p.num_partitions, p.partition_blocks,
                                     p.num_blocks))
        return 1;
    return (L + kBlockSize - 1) / kBlockSize;
}

// Partition `part` of the context of KV head `kvh` of sequence `s`.
template <typename KV, int D, int GMAX, typename OUT, bool WRITE, bool SOLO>
__device__ __forceinline__ void process_partition(const DecodeParams& p, float* smem, int kvh,
                                                  int s, int L, int part) {
    const bool bad = context_unreadable(L, p.table_blocks, p.num_partitions, p.partition_blocks,
                                        p.num_blocks);
    if (bad || L == 0) {
        if (part == 0 && !p.partials_only)
            fill_rows<OUT, SOLO>(p, kvh, s, D, bad ? __builtin_nanf("") : 0.0f);
        return;
    }
    const int nblk = (L + kBlockSize - 1) / kBlockSize;
    const int PB = p.partition_blocks;
    const int np = (nblk + PB - 1) / PB;
    if (part >= np)
        return;
    process_range<KV, D, GMAX, OUT, WRITE, SOLO>(p, smem, kvh, s, L, part * PB, min((part + 1) * PB, nblk),
                                           part, np == 1 && !p.partials_only);
}

// Grid schedule: one workgroup per (KV head, sequence, partition). The single
// pass is the case of one partition spanning the whole table.
template <typename KV, int D, int GMAX, typename OUT, bool WRITE>
__global__ __launch_bounds__(kMaxWaves * kWave) void paged_decode_kernel(DecodeParams p) {
    extern __shared__ float smem[];
    process_partition<KV, D, GMAX, OUT, WRITE, false>(p, smem, blockIdx.x, blockIdx.y,
                                               call_len(p.context_lens[blockIdx.y], p.skip_blocks),
                                               blockIdx.z);
}

// Waves per SIMD the persistent kernel is register-allocated for: three 4-wave
// workgroups per CU for head groups up to 4, two for larger ones.
template <typename KV, int D, int GMAX>
constexpr int persistent_waves_per_simd() {
    return (GMAX <= 4 && D * KV::kBytes <= 256) ? 3 : 2;
}

// #{j < n : a[j] <= x} for a non-decreasing array a (in LDS): a 64-way
// search in which each lane compares one sampled entry and the ballot's
// population count narrows the range to one sampling interval (one step for
// n <= 64, two for n <= 4096). Wave-uniform result. Invariant: a[j] <= x for
// j < base and a[j] > x for j >= base + span.
__device__ __forceinline__ int count_at_most(const int* a, int n, int x, int lane) {
    int base = 0, span = n;
    while (span > kWave) {
        const int stride = (span + kWave - 1) / kWave;
        const int off = lane * stride;
        const bool le = off < span && a[base + off] <= x;
        const int k = __popcll(__ballot(le));      // samples 0 .. k-1 are <= x
        if (k == 0)
            return base;
        base += (k - 1) * stride + 1;
        span = min(stride - 1, span - (k - 1) * stride - 1);
    }
    const bool le = lane < span && a[base + lane] <= x;
    return base + __popcll(__ballot(le));
}

// Persistent schedule: W workgroups, no more than the GPU holds at once, and
// their waves are the workers: V = W * NW of them. The (sequence, partition,
// KV head) items that exist are numbered, KV head fastest, through prefix sums
// of per-sequence counts that each workgroup builds in LDS from context_lens
// (so no worker is spent on the empty partitions of short sequences). For up
// to kMaxSortedSeqs sequences the order is: every full partition (sequence by
// sequence), then the sequences' last, partly filled partitions in
// kSizeClasses classes of their block count, largest first; for larger
// batches, sequence by sequence. Item i goes to worker i mod V in even passes
// over the workers and to V - 1 - (i mod V) in odd ones, so that a worker
// that drew a long item early draws a short one late: with several items per
// wave the busiest wave ends close to the mean. A wave finds each of its
// items itself (count_at_most over the prefix sums) and computes it alone
// (SOLO): after the prefix sums no wave waits for another. With at least as
// many items as workers, wave j of workgroup w is worker v = w * NW + j (a
// workgroup's waves take neighbouring items: the same blocks of neighbouring
// KV heads); with fewer, v = j * W + w, so that the items still spread over
// every CU instead of filling the first workgroups. (Measured on MI355X: one
// wave per item beats a whole workgroup per item -- 201 against 221 us on 8 x
// 32768-token contexts in 512-token partitions, and about as fast on short
// ones; a workgroup per item in turn beat contiguous, tile-balanced ranges,
// and dealing KV head by KV head. The size-class order with alternating
// directions against sequence order in one direction: 838 against 854 us on
// 256 sequences of 1024-8192 tokens in 512-token partitions, 46.1 against
// 47.8-48.6 us for the suffixes and prefix tiles of the shared-prefix batch.
// Building the prefix sums with DPP row shifts and finding items by the
// 64-way search, instead of an item list built in LDS by the whole
// workgroup, brought the moment a wave knows its first item from ~2.5 to
// ~1.4 us after the kernel starts on a 64-sequence batch.)
template <typename KV, int D, int GMAX, typename OUT, bool WRITE>
__device__ __forceinline__ void persistent_items(const DecodeParams& p, float* smem, int* lens, int wg,
                                                 int num_wgs) {
    const int lane = threadIdx.x & (kWave - 1);
    const int S = p.num_seqs, Hkv = p.num_kv_heads, PB = p.partition_blocks;
    const bool sorted = S <= kMaxSortedSeqs;
    // sorted: incl[0][s] full partitions of sequences 0..s, incl[1 + c][s]
    // sequences 0..s whose last partition is partial and of class c;
    // otherwise incl[0][s] partitions of sequences 0..s. Then the totals.
    int* incl = lens + S;
    int* total = incl + (sorted ? 1 + kSizeClasses : 1) * S;
    for (int i = threadIdx.x; i < S; i += blockDim.x)
        lens[i] = call_len(p.context_lens[i], p.skip_blocks);
    __syncthreads();
    if (threadIdx.x < kWave) {
        int cf = 0, c01 = 0, c23 = 0;
        for (int c0 = 0; c0 < S; c0 += kWave) {
            const int i = c0 + lane;
            const int nb = i < S ? schedule_blocks(lens[i], p) : 0;
            int f, p01 = 0, p23 = 0;
            if (sorted) {
                f = nb / PB;
                const int rest = nb - f * PB;
                const int cls = rest > 0 ? (PB - 1 - rest) * kSizeClasses / PB : -1;
                p01 = (cls == 0 ? 1 : 0) | (cls == 1 ? 1 << 16 : 0);
                p23 = (cls == 2 ? 1 : 0) | (cls == 3 ? 1 << 16 : 0);
            } else {
                f = (nb + PB - 1) / PB;
            }
            const int sf = cf + dev::wave_inclusive_sum(f);
            if (i < S)
                incl[i] = sf;
            cf = __builtin_amdgcn_readlane(sf, kWave - 1);
            if (sorted) {
                // Two class counts per 32-bit word: below 2^16 for S <= kMaxSortedSeqs.
                const int s01 = c01 + dev::wave_inclusive_sum(p01);
                const int s23 = c23 + dev::wave_inclusive_sum(p23);
                if (i < S) {
                    incl[S + i] = s01 & 0xFFFF;
                    incl[2 * S + i] = s01 >> 16;
                    incl[3 * S + i] = s23 & 0xFFFF;
                    incl[4 * S + i] = s23 >> 16;
                }
                c01 = __builtin_amdgcn_readlane(s01, kWave - 1);
                c23 = __builtin_amdgcn_readlane(s23, kWave - 1);
            }
        }
        if (lane == 0) {
            total[0] = cf;
            total[1] = c01 & 0xFFFF;
            total[2] = c01 >> 16;
            total[3] = c23 & 0xFFFF;
            total[4] = c23 >> 16;
        }
    }
    __syncthreads();
    const int full = __builtin_amdgcn_readfirstlane(total[0]);
    int slots = full;
    if (sorted) {
#pragma unroll
        for (int c = 0; c < kSizeClasses; ++c)
            slots += __builtin_amdgcn_readfirstlane(total[1 + c]);
    }
    const int64_t items = static_cast<int64_t>(slots) * Hkv;
    const int nw = blockDim.x / kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t V = static_cast<int64_t>(num_wgs) * nw;
    const int64_t v = items >= V ? static_cast<int64_t>(wg) * nw + wave
                                 : static_cast<int64_t>(wave) * num_wgs + wg;
    for (int64_t k = 0;; ++k) {
        const int64_t it = k * V + ((k & 1) ? V - 1 - v : v);
        if (it >= items)
            break;          // only the last pass over the workers is partial
        const int slot = items <= INT32_MAX
                             ? static_cast<int>(static_cast<uint32_t>(it) / static_cast<uint32_t>(Hkv))
                             : static_cast<int>(it / Hkv);
        const int kvh = static_cast<int>(it - static_cast<int64_t>(slot) * Hkv);
        int seq, part;
        if (slot < full) {
            seq = count_at_most(incl, S, slot, lane);
            part = slot - (seq > 0 ? incl[seq - 1] : 0);
        } else {
            int r = slot - full, c = 0;
            while (c < kSizeClasses - 1 && r >= total[1 + c]) {
                r -= total[1 + c];
                ++c;
            }
            seq = count_at_most(incl + (1 + c) * S, S, r, lane);
            part = incl[seq] - (seq > 0 ? incl[seq - 1] : 0);      // its full partitions
        }
        seq = __builtin_amdgcn_readfirstlane(seq);
        process_partition<KV, D, GMAX, OUT, WRITE, true>(p, smem, kvh, seq,
                                                  __builtin_amdgcn_readfirstlane(lens[seq]),
                                                  __builtin_amdgcn_readfirstlane(part));
    }
}

template <typename KV, int D, int GMAX, typename OUT, bool WRITE>
__global__ __launch_bounds__(kPartWaves * kWave)
__attribute__((amdgpu_waves_per_eu(persistent_waves_per_simd<KV, D, GMAX>())))
void paged_decode_persistent_kernel(DecodeParams p) {
    extern __shared__ float smem[];
    int* lens = reinterpret_cast<int*>(smem + decode_lds_floats(KV::kBytes, D, p.group, blockDim.x / kWave));
    persistent_items<KV, D, GMAX, OUT, WRITE>(p, smem, lens, blockIdx.x, gridDim.x);
}

// Shared-prefix batch in one launch: workgroups below tile_wgs take the tiles
// of the shared-prefix product (tile t = KV head fastest, then 64-row tile,
// then prefix chunk; workgroup w takes t = w, w + tile_wgs, ...), the others
// run the persistent schedule over the suffixes. The prefix tiles are bound
// by their loads' latency and the MFMA step, the suffixes by HBM bandwidth,
// so the two kinds of work share the CUs instead of following each other.
// Both write disjoint partial slots of the workspace. The LDS holds either
// kind's working set at its start, the suffixes' context lengths and
// partition prefix sums behind both.
template <int D, int GMAX, typename OUT>
__global__ __launch_bounds__(kPartWaves * kWave)
__attribute__((amdgpu_waves_per_eu(persistent_waves_per_simd<BF16, D, GMAX>())))
void cascade_shared_kernel(DecodeParams p, CascadeParams c, int tile_wgs) {
    extern __shared__ float smem[];
    static_assert(kPartWaves == kCascadeWaves, "both kinds of work use the same workgroup");
    if (static_cast<int>(blockIdx.x) < tile_wgs) {
        auto& lds = *reinterpret_cast<tile::Lds<D, kCascadeWaves>*>(smem);
        const int tiles = c.num_kv_heads * c.row_tiles * c.num_chunks;
        for (int t = blockIdx.x; t < tiles; t += tile_wgs) {
            const int kvh = t % c.num_kv_heads;
            const int r = t / c.num_kv_heads;
            tile::prefix_tile<D>(c, lds, kvh, r % c.row_tiles, r / c.row_tiles);
            __syncthreads();                    // the step's LDS is free for the next tile
        }
        return;
    }
    int* lens = reinterpret_cast<int*>(smem + cascade_shared_area_floats(D, p.group));
    persistent_items<BF16, D, GMAX, OUT, false>(p, smem, lens, blockIdx.x - tile_wgs,
                                                gridDim.x - tile_wgs);
}

// Log-sum-exp combination of the partitions of every (sequence, KV head)
// whose context spans more than one partition: one workgroup per (sequence,
// KV head), one wave per query head of the group. The row's partials are its
// own partitions followed by any extra slots (shared-prefix chunks), merged
// 64 at a time:
//     M = max_i m_i,  w_i = s_i exp(m_i - M),  out = sum_i w_i o_i / sum_i w_i,
// the running sums rescaled when a later batch raises M. The loads of a batch
// (maxima, sums and the output rows of up to 16 partials) are all issued
// before any of them is used; further output rows follow 32 at a time. A
// partial's slot is computed from its index (no table); a batch's maximum and
// weight sum are wave reductions in the VALU (DPP within 16-lane rows, then
// row swaps), with no LDS round trip. All reductions run in a fixed order
// (the outputs partial by partial), whatever the batching.
template <int D, typename OUT>
__global__ __launch_bounds__(kReduceMaxWaves * kWave) void lse_reduce_kernel(ReduceParams p) {
    constexpr int DPL = D / kWave;              // output elements per lane
    constexpr int PRE = 16;                     // partial outputs loaded with the statistics
    constexpr int MORE = 32;                    // partial outputs loaded together after those
    const int kvh = blockIdx.x;
    const int s = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    const int G = p.group, Hq = p.num_q_heads, NP = p.num_partitions;
    const int L = call_len(p.context_lens[s], p.skip_blocks);
    const bool bad = context_unreadable(L, p.table_blocks, NP, p.partition_blocks, p.num_blocks);
    if (p.extra_count == 0 && (bad || L == 0))
        return;                                // the decode kernel wrote this row
    if (bad) {                                 // cascade: an unreadable suffix
        for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
            const int h = idx / D, d = idx - (idx / D) * D;
            store_out<OUT>(p.out, ((int64_t)s * Hq + kvh * G + h) * D + d, __builtin_nanf(""));
        }
        return;
    }
    const int nblk = (L + kBlockSize - 1) / kBlockSize;
    const int own = (nblk + p.partition_blocks - 1) / p.partition_blocks;   // 0 when L == 0
    if (p.extra_count == 0 && own <= 1)
        return;                                // written directly by its only partition
    const int total = own + p.extra_count;     // partial slots: own partitions, then extras
    auto slot_of = [&](int i) { return i < own ? i : p.extra_base + (i - own); };
    for (int h = wave; h < G; h += nw) {
        const int64_t row = (int64_t)s * Hq + (int64_t)kvh * G + h;
        const int64_t base = row * p.part_stride;
        float M = -INFINITY, T = 0.0f;
        float acc[DPL];
#pragma unroll
        for (int e = 0; e < DPL; ++e)
            acc[e] = 0.0f;
        for (int c0 = 0; c0 < total; c0 += kWave) {
            const int i = c0 + lane;
            const int n = min(kWave, total - c0);
            // Lane j < n holds partial j's statistics; the first PRE outputs are
            // requested together with them.
            const int my = lane < n ? slot_of(i) : 0;
            const float mv = lane < n ? p.part_max[base + my] : -INFINITY;
            const float sv = lane < n ? p.part_sum[base + my] : 0.0f;
            float ov[PRE][DPL];
#pragma unroll
            for (int j = 0; j < PRE; ++j) {
                // Past the batch's partials the load re-reads slot 0 of the row
                // (always inside the workspace); the value is not used.
                const int sj = j < n ? slot_of(c0 + j) : 0;
                const float* po = p.part_out + (base + sj) * D + lane;
#pragma unroll
                for (int e = 0; e < DPL; ++e)
                    ov[j][e] = po[e * kWave];
            }
            const float cm = dev::wave_max(mv);
            const float Mn = fmaxf(M, cm);
            const float scale = M == Mn ? 1.0f : __builtin_amdgcn_exp2f((M - Mn) * kLog2e);
            const float wv = lane < n ? sv * __builtin_amdgcn_exp2f((mv - Mn) * kLog2e) : 0.0f;
            const float ws = dev::wave_sum(wv);
            T = T * scale + ws;
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                acc[e] *= scale;
#pragma unroll
            for (int j = 0; j < PRE; ++j) {
                if (j < n) {
                    const float w = readlane_f(wv, j);
#pragma unroll
                    for (int e = 0; e < DPL; ++e)
                        acc[e] = fmaf(w, ov[j][e], acc[e]);
                }
            }
            // The batch's remaining partials, MORE at a time, each group's
            // loads in flight together.
            for (int j0 = PRE; j0 < n; j0 += MORE) {
                float om[MORE][DPL];
#pragma unroll
                for (int j = 0; j < MORE; ++j) {
                    const int sj = j0 + j < n ? slot_of(c0 + j0 + j) : 0;
                    const float* po = p.part_out + (base + sj) * D + lane;
#pragma unroll
                    for (int e = 0; e < DPL; ++e)
                        om[j][e] = po[e * kWave];
                }
#pragma unroll
                for (int j = 0; j < MORE; ++j) {
                    if (j0 + j < n) {
                        const float w = readlane_f(wv, j0 + j);
#pragma unroll
                        for (int e = 0; e < DPL; ++e)
                            acc[e] = fmaf(w, om[j][e], acc[e]);
                    }
                }
            }
            M = Mn;
        }
#pragma unroll
        for (int e = 0; e < DPL; ++e)
            store_out<OUT>(p.out, row * D + lane + e * kWave, acc[e] / T);
    }
}

template <typename KV, int D, int GMAX, typename OUT, bool WRITE>
hipError_t launch_decode_grid(const DecodeParams& p, int num_seqs, int grid_partitions, int waves,
                              hipStream_t stream) {
    const size_t lds = decode_lds_bytes(KV::kBytes, D, p.group, waves);
    hipLaunchKernelGGL((paged_decode_kernel<KV, D, GMAX, OUT, WRITE>),
                       dim3(p.num_kv_heads, num_seqs, grid_partitions), dim3(waves * kWave), lds,
                       stream, p);
    return hipGetLastError();
}

template <typename KV, int D, int GMAX, typename OUT, bool WRITE>
hipError_t launch_decode_w(const DecodeParams& p, int num_seqs, int grid_partitions, int waves,
                           hipStream_t stream) {
    if (!p.persistent)
        return launch_decode_grid<KV, D, GMAX, OUT, WRITE>(p, num_seqs, grid_partitions, waves, stream);
    const auto kernel = paged_decode_persistent_kernel<KV, D, GMAX, OUT, WRITE>;
    // Persistent: as many kPartWaves-wave workgroups as the GPU keeps resident
    // at once (never more waves than there can be items); each wave takes its
    // own items, so the workgroup size does not follow the partition size.
    const size_t lds = decode_lds_bytes(KV::kBytes, D, p.group, kPartWaves) + persistent_lds_bytes(num_seqs);
    int dev = 0, per_cu = 0;
    DeviceInfo info{};
    hipError_t e = current_device_info(&dev, &info);
    if (e != hipSuccess)
        return e;
    if (lds > static_cast<size_t>(info.max_lds)) {
        // The context lengths do not fit one workgroup's LDS: one workgroup
        // per (KV head, sequence, partition) computes the same partials.
        DecodeParams g = p;
        g.persistent = 0;
        return launch_decode_grid<KV, D, GMAX, OUT, WRITE>(g, num_seqs, grid_partitions, waves, stream);
    }
    e = resident_workgroups_per_cu(dev, reinterpret_cast<const void*>(kernel), kPartWaves * kWave, lds,
                                   &per_cu);
    if (e != hipSuccess)
        return e;
    const int64_t bound = (static_cast<int64_t>(num_seqs) * p.num_kv_heads * grid_partitions + kPartWaves - 1) /
                          kPartWaves;
    const int64_t wgs = std::max<int64_t>(1, std::min<int64_t>(bound, static_cast<int64_t>(info.cus) *
                                                                         std::max(per_cu, 1)));
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(wgs)), dim3(kPartWaves * kWave), lds, stream, p);
    return hipGetLastError();
}

template <typename KV, int D, int GMAX, typename OUT>
hipError_t launch_decode_t(const DecodeParams& p, int num_seqs, int grid_partitions, int waves,
                           hipStream_t stream) {
    return p.new_key ? launch_decode_w<KV, D, GMAX, OUT, true>(p, num_seqs, grid_partitions, waves, stream)
                     : launch_decode_w<KV, D, GMAX, OUT, false>(p, num_seqs, grid_partitions, waves, stream);
}

template <typename KV, int D, typename OUT>
hipError_t launch_decode_g(const DecodeParams& p, int num_seqs, int grid_partitions, int waves,
                           hipStream_t stream) {
    switch (decode_gmax(p.group)) {
    case 1: return launch_decode_t<KV, D, 1, OUT>(p, num_seqs, grid_partitions, waves, stream);
    case 2: return launch_decode_t<KV, D, 2, OUT>(p, num_seqs, grid_partitions, waves, stream);
    case 4: return launch_decode_t<KV, D, 4, OUT>(p, num_seqs, grid_partitions, waves, stream);
    case 8: return launch_decode_t<KV, D, 8, OUT>(p, num_seqs, grid_partitions, waves, stream);
    default: return launch_decode_t<KV, D, 16, OUT>(p, num_seqs, grid_partitions, waves, stream);
    }
}

template <typename KV, int D>
hipError_t launch_decode_o(const DecodeParams& p, int out_bf16, int num_seqs, int grid_partitions,
                           int waves, hipStream_t stream) {
    return out_bf16 ? launch_decode_g<KV, D, BF16>(p, num_seqs, grid_partitions, waves, stream)
                    : launch_decode_g<KV, D, F32>(p, num_seqs, grid_partitions, waves, stream);
}

template <int D, int GMAX, typename OUT>
hipError_t launch_cascade_shared_t(const DecodeParams& p, const CascadeParams& c, int num_seqs,
                                   int grid_partitions, bool* launched, hipStream_t stream) {
    const auto kernel = cascade_shared_kernel<D, GMAX, OUT>;
    const size_t lds = sizeof(float) * cascade_shared_area_floats(D, p.group) + persistent_lds_bytes(num_seqs);
    int dev = 0, per_cu = 0;
    DeviceInfo info{};
    *launched = false;
    hipError_t e = current_device_info(&dev, &info);
    if (e != hipSuccess || lds > static_cast<size_t>(info.max_lds))
        return e;
    e = resident_workgroups_per_cu(dev, reinterpret_cast<const void*>(kernel), kPartWaves * kWave, lds,
                                   &per_cu);
    if (e != hipSuccess)
        return e;
    // One tile per tile workgroup, one tile workgroup per CU at most; the
    // rest of the resident grid (at least one workgroup, never more than
    // there can be suffix items) decodes. On the 128-sequence batch with a
    // 2048-token prefix, 64-block tiles (128 of them, 32 steps each) measured
    // 46.5 us per call; 32-block tiles 52.4 us at one per workgroup, 50.1 us
    // at two, 71.2 us at four (the tiles then finish last).
    const int tiles = c.num_kv_heads * c.row_tiles * c.num_chunks;
    const int tile_wgs = std::min(tiles, info.cus);
    const int64_t resident = static_cast<int64_t>(info.cus) * std::max(per_cu, 1);
    const int64_t bound = (static_cast<int64_t>(num_seqs) * p.num_kv_heads * grid_partitions + kPartWaves - 1) /
                          kPartWaves;
    const int64_t decode_wgs = std::max<int64_t>(1, std::min<int64_t>(bound, resident - tile_wgs));
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(tile_wgs + decode_wgs)), dim3(kPartWaves * kWave),
                       lds, stream, p, c, tile_wgs);
    e = hipGetLastError();
    *launched = e == hipSuccess;
    return e;
}

template <int D, typename OUT>
hipError_t launch_cascade_shared_g(const DecodeParams& p, const CascadeParams& c, int num_seqs,
                                   int grid_partitions, bool* launched, hipStream_t stream) {
    switch (decode_gmax(p.group)) {
    case 1: return launch_cascade_shared_t<D, 1, OUT>(p, c, num_seqs, grid_partitions, launched, stream);
    case 2: return launch_cascade_shared_t<D, 2, OUT>(p, c, num_seqs, grid_partitions, launched, stream);
    case 4: return launch_cascade_shared_t<D, 4, OUT>(p, c, num_seqs, grid_partitions, launched, stream);
    case 8: return launch_cascade_shared_t<D, 8, OUT>(p, c, num_seqs, grid_partitions, launched, stream);
    default: return launch_cascade_shared_t<D, 16, OUT>(p, c, num_seqs, grid_partitions, launched, stream);
    }
}

}  // namespace

hipError_t launch_reduce(const ReduceParams& p, int head_size, int out_bf16, int num_seqs,
                         hipStream_t stream) {
    const dim3 grid(p.num_kv_heads, num_seqs);
    const dim3 block(std::min(p.group, kReduceMaxWaves) * kWave);
    if (head_size == 64) {
        if (out_bf16)
            hipLaunchKernelGGL((lse_reduce_kernel<64, BF16>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((lse_reduce_kernel<64, F32>), grid, block, 0, stream, p);
    } else {
        if (out_bf16)
            hipLaunchKernelGGL((lse_reduce_kernel<128, BF16>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((lse_reduce_kernel<128, F32>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int kv_bf16, int head_size, int out_bf16,
                         int num_seqs, int grid_partitions, int waves, hipStream_t stream) {
    if (kv_bf16) {
        return head_size == 64
                   ? launch_decode_o<BF16, 64>(p, out_bf16, num_seqs, grid_partitions, waves, stream)
                   : launch_decode_o<BF16, 128>(p, out_bf16, num_seqs, grid_partitions, waves, stream);
    }
    return head_size == 64
               ? launch_decode_o<F32, 64>(p, out_bf16, num_seqs, grid_partitions, waves, stream)
               : launch_decode_o<F32, 128>(p, out_bf16, num_seqs, grid_partitions, waves, stream);
}

hipError_t launch_cascade_shared(const DecodeParams& p, const CascadeParams& c, int head_size,
                                 int out_bf16, int num_seqs, int grid_partitions, bool* launched,
                                 hipStream_t stream) {
    if (head_size == 64)
        return out_bf16 ? launch_cascade_shared_g<64, BF16>(p, c, num_seqs, grid_partitions, launched, stream)
                        : launch_cascade_shared_g<64, F32>(p, c, num_seqs, grid_partitions, launched, stream);
    return out_bf16 ? launch_cascade_shared_g<128, BF16>(p, c, num_seqs, grid_partitions, launched, stream)
                    : launch_cascade_shared_g<128, F32>(p, c, num_seqs, grid_partitions, launched, stream);
}

}  // namespace pa

// pa_prefill.hip -- multi-token queries over the paged KV cache (a prompt, or
// a chunk of one, whose keys and values are already in the cache), for
// gfx950 (CDNA4).
//
// "Problem 1" on "vLLM Solved the Wrong Bottleneck" follows a prompt of many
// tokens and then each generated token, every one of which needs the keys
// and values of all tokens before it; the paged cache holds those keys and
// values in blocks ("The idea vLLM started from: pages" on "What vLLM Is and
// Why It Exists"). Reading (the pages give no formula for the prompt phase):
// a sequence s brings q_s query rows, the last q_s tokens of its context of
// L_s tokens; row i sits at position L_s - q_s + i and attends, causally, to
// tokens 0 .. L_s - q_s + i, read through the block table. With q_s = 1 this
// is the decode step; with q_s = L_s it is a whole prompt.
//
// Work decomposition: one workgroup per (128-row tile, KV head, sequence),
// where the rows of a (sequence, KV head) are its (query token, head of the
// group) pairs, token-major, so that a tile spans 128 / G consecutive query
// tokens and the K/V it reads is shared by all its rows: a dense tile for
// MFMA. Workgroups run from 1 to hundreds of steps (the later tiles of long
// contexts the most), so a one-workgroup kernel first orders the (sequence,
// tile) pairs by their step counts, most first, and the workgroups take the
// pairs in that order (longest work dispatched first). Per workgroup, 4 waves of two 16-row MFMA tiles each, one
// step of 32 context tokens (two blocks) at a time, the step of pa_tile.h:
// K and V^T staged in LDS (two buffers, one barrier per step), K Q^T and
// V^T P^T on v_mfma_f32_16x16x32_bf16 with P kept in registers (split into a
// bf16 high part and remainder), online softmax per row with its statistics
// in the row's four lanes; the causal mask is a select per row (token <= the
// row's position), and V of tokens past the tile's last position (the block
// tail, which may hold anything) is staged as zeros. The next step's K and V
// are requested before this step computes. Block ids come from a per-lane
// register holding 64 consecutive table entries, reloaded every 64 blocks.
#include "pa_tile.h"

namespace pa {
namespace {

using namespace dev;

template <typename OUT>
__device__ __forceinline__ void store_row_value(void* out, int64_t idx, float v);
template <>
__device__ __forceinline__ void store_row_value<F32>(void* out, int64_t idx, float v) {
    static_cast<float*>(out)[idx] = v;
}
template <>
__device__ __forceinline__ void store_row_value<BF16>(void* out, int64_t idx, float v) {
    static_cast<uint16_t*>(out)[idx] = bf16_out(v);
}

// Steps (of 32 tokens) the workgroup of row tile `tile` of sequence s runs:
// 0 when it has no rows or its rows cannot be computed. Mirrors the bounds
// of prefill_kernel.
__device__ __forceinline__ int prefill_steps(const PrefillParams& p, int s, int tile) {
    constexpr int TROWS = kPrefillWaves * 16 * kPrefillRowTiles;
    const int q0 = p.query_start[s];
    const int64_t q_end = p.query_start[s + 1];
    if (q0 < 0 || q_end > p.num_query_rows)
        return 0;
    const int nq = q_end > q0 ? static_cast<int>(q_end - q0) : 0;
    const int rows = min(nq, p.max_query_len) * p.group;
    const int tile0 = tile * TROWS;
    const int L = p.context_lens[s];
    if (tile0 >= rows || nq > L || static_cast<int64_t>(L) > static_cast<int64_t>(p.max_blocks_per_seq) * kBlockSize)
        return 0;
    const int last_row = min(tile0 + TROWS, rows) - 1;
    const int maxpos = L - nq + last_row / p.group;
    return (maxpos / kBlockSize + 2) / 2;
}

// Orders the (sequence, row tile) pairs: sequences by the steps of their
// longest row tile, most first (a counting sort over those step counts in
// LDS; sequences with equal counts in any order), and each sequence's row
// tiles together, its last (longest) tile first. The dispatcher then starts
// the longest work first, and the tiles of one sequence run at about the same
// time on their KV head's XCD, where they share the sequence's K and V in L2.
// A pair's rows are computed the same way wherever it lands, so the order
// never changes a result. One workgroup.
__global__ __launch_bounds__(1024) void prefill_order_kernel(PrefillParams p, int num_seqs) {
    constexpr int NB = kPrefillOrderBins;
    constexpr int PER = NB / 1024;             // bins per thread in the scan
    constexpr int NW = 1024 / kWave;
    __shared__ int hist[NB];
    __shared__ int start[NB];
    __shared__ int wave_total[NW];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const int RT = p.row_tiles;
    for (int i = tid; i < NB; i += 1024)
        hist[i] = 0;
    auto bin_of = [&](int s) {
        int most = 0;                          // row tiles' steps do not decrease with the tile
        for (int t = RT - 1; t >= 0 && most == 0; --t)
            most = prefill_steps(p, s, t);
        // Bin 0 holds the most steps: the order is ascending in bins.
        return NB - 1 - min(most, NB - 1);
    };
    const int my_bin = tid < num_seqs ? bin_of(tid) : 0;     // kept for the scatter below
    __syncthreads();
    for (int s = tid; s < num_seqs; s += 1024)
        atomicAdd(&hist[s == tid ? my_bin : bin_of(s)], 1);
    __syncthreads();
    // Exclusive prefix sum of hist: each thread sums PER consecutive bins, a
    // DPP scan within each wave, then one over the waves' totals.
    int local = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k)
        local += hist[tid * PER + k];
    const int incl = dev::wave_inclusive_sum(local);
    if (lane == kWave - 1)
        wave_total[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const int t = lane < NW ? wave_total[lane] : 0;
        const int ti = dev::wave_inclusive_sum(t);
        if (lane < NW)
            wave_total[lane] = ti - t;         // exclusive: the bins before this wave's
    }
    __syncthreads();
    int run = wave_total[wave] + incl - local;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        start[tid * PER + k] = run;
        run += hist[tid * PER + k];
    }
    __syncthreads();
    for (int s = tid; s < num_seqs; s += 1024) {
        const int64_t r = atomicAdd(&start[s == tid ? my_bin : bin_of(s)], 1);    // the sequence's rank
        for (int j = 0; j < RT; ++j)
            p.order[r * RT + j] = s * RT + (RT - 1 - j);
    }
}

template <int D, typename OUT>
__global__ __launch_bounds__(kPrefillWaves * kWave)
__attribute__((amdgpu_waves_per_eu(2)))
void prefill_kernel(PrefillParams p) {
    using S = tile::Shape<D, kPrefillWaves>;
    constexpr int ROW = S::ROW, NQ = S::NQ, NT = S::NT, RT = kPrefillRowTiles;
    constexpr int TROWS = kPrefillWaves * 16 * RT;   // rows per workgroup
    __shared__ __attribute__((aligned(16))) tile::Lds<D, kPrefillWaves> lds;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int g = lane >> 4;
    const int r16 = lane & 15;
    // Workgroups go out in blockIdx order, so taking the (sequence, row tile)
    // pairs in the order prefill_order_kernel wrote (most steps first, the KV
    // heads of a pair adjacent) hands the longest work out first.
    const int G = p.group, Hq = p.num_q_heads, Hkv = p.num_kv_heads;
    const int pair = p.order[blockIdx.x / Hkv];
    const int kvh = static_cast<int>(blockIdx.x % Hkv);
    const int s = pair / p.row_tiles;
    const int tile = pair - s * p.row_tiles;
    const int q0 = p.query_start[s];
    const int64_t q_end = p.query_start[s + 1];
    // Rows outside [0, T) are never touched: such a sequence is skipped whole.
    // A decreasing pair of offsets brings no rows.
    if (q0 < 0 || q_end > p.num_query_rows)
        return;
    const int nq = q_end > q0 ? static_cast<int>(q_end - q0) : 0;
    // Rows computed: the first min(nq, max_query_len) query tokens, every head
    // of the group (none when the sequence brings no rows).
    const int rows = min(nq, p.max_query_len) * G;
    const int tile0 = tile * TROWS;
    if (tile0 >= rows)
        return;
    const int L = p.context_lens[s];
    const int64_t cap = static_cast<int64_t>(p.max_blocks_per_seq) * kBlockSize;
    const int last_row = min(tile0 + TROWS, rows) - 1;
    // Output row of tile row r (r < rows): query token r / G, head r % G.
    auto out_row = [&](int r) {
        return (static_cast<int64_t>(q0) + r / G) * Hq + static_cast<int64_t>(kvh) * G + r % G;
    };
    if (nq > L || static_cast<int64_t>(L) > cap || p.num_blocks <= 0) {
        // Rows that cannot be computed (more query rows than context, or a
        // context longer than its table, or an empty pool): NaN.
        for (int idx = threadIdx.x; idx < (last_row - tile0 + 1) * D; idx += blockDim.x)
            store_row_value<OUT>(p.out, out_row(tile0 + idx / D) * D + idx % D, __builtin_nanf(""));
        return;
    }
    const int32_t* table = p.block_tables + static_cast<int64_t>(s) * p.max_blocks_per_seq;
    // An id outside the pool anywhere in the context poisons the sequence's
    // rows (NaN); every load then reads block 0 instead.
    bool poisoned = false;
    {
        const int nb_ctx = (L + kBlockSize - 1) / kBlockSize;
        bool bad = false;
        for (int b = lane; b < nb_ctx; b += kWave) {
            const int e = table[b];
            bad = bad || e < 0 || static_cast<int64_t>(e) >= p.num_blocks;
        }
        poisoned = __ballot(bad) != 0;
    }

    // Rows of this wave: tile t holds rows row0 + 16t + r16 (lane row r16).
    const int row0 = tile0 + wave * 16 * RT;
    u32x4 qa[RT][NQ];
    int pos[RT];                                // causal limit of row r16 of tile t
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int r = row0 + 16 * t + r16;
        const bool live = r < rows;
        const char* qp = static_cast<const char*>(p.q) + out_row(live ? r : tile0) * ROW;
#pragma unroll
        for (int c = 0; c < NQ; ++c)
            qa[t][c] = live ? *reinterpret_cast<const u32x4*>(qp + (g + 4 * c) * 16)
                            : u32x4{0u, 0u, 0u, 0u};
        pos[t] = live ? L - nq + r / G : 0;
    }
    // The smallest causal limit among each tile's rows (its first row, or 0
    // when some of its rows are past the last): a step whose 32 tokens all
    // lie at or below it needs no mask.
    int pos_min[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int r_first = row0 + 16 * t, r_last = row0 + 16 * t + 15;
        pos_min[t] = r_last < rows ? L - nq + r_first / G : -1;
    }
    const int maxpos = L - nq + last_row / G;   // the tile reads tokens 0 .. maxpos
    const int nblk = maxpos / kBlockSize + 1;
    const int nsteps = (nblk + 1) / 2;

    const char* kbase = static_cast<const char*>(p.k_cache) + (int64_t)kvh * S::TILE;
    const char* vbase = static_cast<const char*>(p.v_cache) + (int64_t)kvh * S::TILE;
    const int64_t blk_stride = (int64_t)Hkv * S::TILE;

    // Table entries: lane i holds block ids_base + i.
    int ids = 0, ids_base = -kWave;
    auto id_of = [&](int b) {
        if (b >= ids_base + kWave) {            // wave-uniform
            ids_base = b & ~(kWave - 1);
            const int jb = ids_base + lane;
            const int e = jb < nblk ? table[jb] : 0;
            ids = (e < 0 || static_cast<int64_t>(e) >= p.num_blocks) ? 0 : e;
        }
        return __builtin_amdgcn_readlane(ids, b - ids_base);
    };
    tile::Loader<D, kPrefillWaves> ld;
    ld.init();
    tile::RowState<D, RT> rs;
    rs.reset();
    // A lone last block is read twice; its second copy lies past maxpos.
    tile::run_steps<D, kPrefillWaves>(
        nsteps,
        [&](tile::StepData<D, kPrefillWaves>& d, int st) {
            const int id0 = id_of(2 * st);
            const int id1 = id_of(min(2 * st + 1, nblk - 1));
            ld.load(d, kbase, vbase, blk_stride, id0, id1);
        },
        [&](const tile::StepData<D, kPrefillWaves>& d, int st, int buf) {
            ld.stage(d, lds, buf, maxpos - st * tile::kStepTokens + 1);
        },
        [&](int st, int buf) {
            const int t0 = st * tile::kStepTokens;
            tile::attend<D, kPrefillWaves, RT>(lds, buf, qa, p.scale_log2,
                                               [&](int t, int tok) { return t0 + tok <= pos[t]; },
                                               [&](int t) { return t0 + tile::kStepTokens - 1 <= pos_min[t]; },
                                               rs);
        });

    // Output row r16 of each tile, columns 16n + 4g + j.
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const float srow = rs.row_sum(t);
        const int r = row0 + 16 * t + r16;
        if (r >= rows)
            continue;
        const int64_t base = out_row(r) * D;
        const float inv = 1.0f / srow;
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                store_row_value<OUT>(p.out, base + n * 16 + 4 * g + j,
                                     poisoned ? __builtin_nanf("") : rs.o[t][n][j] * inv);
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int head_size, int out_bf16, int num_seqs,
                          int row_tiles, hipStream_t stream) {
    PrefillParams q = p;
    q.row_tiles = row_tiles;
    const int num_pairs = num_seqs * row_tiles;
    hipLaunchKernelGGL(prefill_order_kernel, dim3(1), dim3(1024), 0, stream, q, num_seqs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(num_pairs) * p.num_kv_heads));
    const dim3 block(kPrefillWaves * kWave);
    if (head_size == 64) {
        if (out_bf16)
            hipLaunchKernelGGL((prefill_kernel<64, BF16>), grid, block, 0, stream, q);
        else
            hipLaunchKernelGGL((prefill_kernel<64, F32>), grid, block, 0, stream, q);
    } else {
        if (out_bf16)
            hipLaunchKernelGGL((prefill_kernel<128, BF16>), grid, block, 0, stream, q);
        else
            hipLaunchKernelGGL((prefill_kernel<128, F32>), grid, block, 0, stream, q);
    }
    return hipGetLastError();
}

}  // namespace pa

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
// MFMA. The row tiles of one (sequence, KV head) run on one XCD, so that its
// L2 serves their shared K/V, and successive (sequence, KV head) pairs go to
// different XCDs. Per workgroup, 4 waves of two 16-row MFMA tiles each (the K
// loads, the V transpose and the barriers of a step serve 32 rows of a wave),
// per step of 32 context tokens (two blocks):
//   * the step's K is loaded once per workgroup (each thread a share of its
//     16-byte chunks) into LDS, rows XOR-swizzled so that reads in the MFMA
//     B-operand layout are free of bank conflicts; Q^T K on
//     v_mfma_f32_16x16x32_bf16 gives logits[row][token];
//   * the causal mask is a select per row (token <= the row's position);
//   * online softmax per row (running max and sum, base 2);
//   * P goes through LDS into the A-operand layout, split into a bf16 high
//     part and a bf16 remainder (about 16 bits of P are kept);
//   * V is written to LDS transposed; tokens past the tile's last position
//     (the block tail, which may hold anything) are written as zeros, so that
//     they contribute exactly nothing to P.V on MFMA;
//   * K and V^T live in two LDS buffers used on alternate steps, so one
//     barrier per step suffices;
//   * the next step's K and V are requested before this step computes.
// Block ids come from a per-lane register holding 64 consecutive table
// entries, reloaded every 64 blocks.
#include "pa_device.h"

namespace pa {
namespace {

using namespace dev;

constexpr int kStepTokens = 32;                 // two blocks per step
constexpr int kVtStride = kStepTokens + 8;      // bf16 per transposed V row (80 bytes)
constexpr int kPStride = kStepTokens + 4;       // floats per P row in LDS (144 bytes)

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

template <int D, typename OUT>
__global__ __launch_bounds__(kPrefillWaves * kWave)
__attribute__((amdgpu_waves_per_eu(2)))   // 2 waves per SIMD: 234 VGPRs, no spill (D = 128)
void prefill_kernel(PrefillParams p) {
    constexpr int ROW = D * 2;                  // bytes per token row (bf16)
    constexpr int TILE = kBlockSize * ROW;
    constexpr int CH = ROW / 16;                // 16-byte chunks per row
    constexpr int NQ = CH / 4;                  // K chunks per lane per tile
    constexpr int NT = D / 16;                  // 16-column output tiles
    constexpr int VITEMS = (kStepTokens / 2) * CH;   // (token pair, chunk) items of a step
    constexpr int RT = kPrefillRowTiles;             // 16-row tiles per wave
    constexpr int TROWS = kPrefillWaves * 16 * RT;   // rows per workgroup
    static_assert(VITEMS <= kPrefillWaves * kWave && (kPrefillWaves * kWave) % VITEMS == 0,
                  "one V item per thread");

    constexpr int KITEMS = kStepTokens * CH;         // 16-byte K chunks of a step
    constexpr int KPT = KITEMS / (kPrefillWaves * kWave);   // K chunks per thread
    static_assert(KPT >= 1 && KITEMS % (kPrefillWaves * kWave) == 0, "whole K chunks per thread");
    // K and V^T of a step, two buffers each, alternating per step: a buffer is
    // written again two steps later, after a barrier that every wave passes
    // only once done with it. K rows are kept with their 16-byte chunks
    // XOR-swizzled by the row (chunk j of token t at slot j ^ (t mod CH)), so
    // that the B-operand reads (16 tokens, one chunk) hit 16 different banks.
    __shared__ __attribute__((aligned(16))) u32x4 kl[2][KITEMS];
    __shared__ __attribute__((aligned(16))) uint16_t vt2[2][D][kVtStride];
    __shared__ __attribute__((aligned(16))) float pl[kPrefillWaves][16 * RT][kPStride];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int g = lane >> 4;
    const int r16 = lane & 15;
    // Logical tile: the row tiles of one (sequence, KV head) form a group that
    // runs on one XCD, whose L2 then serves their shared K/V.
    const int64_t nwg = static_cast<int64_t>(gridDim.x) * gridDim.y * gridDim.z;
    const int64_t lid = xcd_grouped(
        blockIdx.x + static_cast<int64_t>(gridDim.x) * (blockIdx.y + static_cast<int64_t>(gridDim.y) * blockIdx.z),
        nwg, gridDim.x);
    const int tile = static_cast<int>(lid % gridDim.x);
    const int kvh = static_cast<int>((lid / gridDim.x) % gridDim.y);
    const int s = static_cast<int>(lid / (static_cast<int64_t>(gridDim.x) * gridDim.y));
    const int G = p.group, Hq = p.num_q_heads, Hkv = p.num_kv_heads;
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

    // Rows of this wave: tile t holds rows row0 + 16t + (A-operand row r16,
    // output rows 4g + j).
    const int row0 = tile0 + wave * 16 * RT;
    u32x4 qa[RT][NQ];
    int pos[RT][4];                             // causal limit of rows 4g + j of tile t
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int r = row0 + 16 * t + r16;
        const bool live = r < rows;
        const char* qp = static_cast<const char*>(p.q) + out_row(live ? r : tile0) * ROW;
#pragma unroll
        for (int c = 0; c < NQ; ++c)
            qa[t][c] = live ? *reinterpret_cast<const u32x4*>(qp + (g + 4 * c) * 16)
                            : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rr = row0 + 16 * t + 4 * g + j;
            pos[t][j] = rr < rows ? L - nq + rr / G : 0;
        }
    }
    const int maxpos = L - nq + last_row / G;   // the tile reads tokens 0 .. maxpos
    const int nblk = maxpos / kBlockSize + 1;
    const int nsteps = (nblk + 1) / 2;

    const char* kbase = static_cast<const char*>(p.k_cache) + (int64_t)kvh * TILE;
    const char* vbase = static_cast<const char*>(p.v_cache) + (int64_t)kvh * TILE;
    const int64_t blk_stride = (int64_t)Hkv * TILE;
    // V item of this thread: token pair tp (tokens 2tp, 2tp + 1 of the step), chunk vc.
    const int vi = threadIdx.x % VITEMS;
    const int tp = vi % (kStepTokens / 2), vc = vi / (kStepTokens / 2);
    const int vblk = tp >> 3;                   // which block of the step
    const int voff = (2 * tp - 16 * vblk) * ROW + vc * 16;

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

    // K chunks of this thread: item q = threadIdx.x + k * threads is chunk
    // q % CH of token q / CH of the step (block (q / CH) / 16, the same for a
    // whole wave), stored at its swizzled slot.
    int kslot[KPT], koff[KPT], kblk[KPT];
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
        const int q = threadIdx.x + k * kPrefillWaves * kWave;
        const int t = q / CH, j = q % CH;
        kslot[k] = t * CH + (j ^ (t & (CH - 1)));
        kblk[k] = t >> 4;
        koff[k] = (t & 15) * ROW + j * 16;
    }
    // Loads of step st: this thread's K chunks of its two blocks (a lone last
    // block is read twice; its second copy lies past maxpos and is masked) and
    // its V pair.
    u32x4 kq[KPT], vr[2];
    auto load_step = [&](int st) {
        const int id0 = id_of(2 * st);
        const int id1 = id_of(min(2 * st + 1, nblk - 1));
#pragma unroll
        for (int k = 0; k < KPT; ++k)
            kq[k] = *reinterpret_cast<const u32x4*>(kbase + (int64_t)(kblk[k] ? id1 : id0) * blk_stride +
                                                    koff[k]);
        const char* v = vbase + (int64_t)(vblk ? id1 : id0) * blk_stride + voff;
        vr[0] = *reinterpret_cast<const u32x4*>(v);
        vr[1] = *reinterpret_cast<const u32x4*>(v + ROW);
    };

    float m[RT][4], lsum[RT][4];
    f32x4 o[RT][NT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            m[t][j] = -INFINITY;
            lsum[t][j] = 0.0f;
        }
#pragma unroll
        for (int n = 0; n < NT; ++n)
            o[t][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    load_step(0);
    for (int st = 0; st < nsteps; ++st) {
        const int t0 = st * kStepTokens;
        const int buf = st & 1;
        auto& vt = vt2[buf];
        // K of the step into LDS; V transposed into LDS (two adjacent tokens
        // per 32-bit word), tokens past maxpos written as zeros.
#pragma unroll
        for (int k = 0; k < KPT; ++k)
            kl[buf][kslot[k]] = kq[k];
        {
            const bool za = t0 + 2 * tp > maxpos, zb = t0 + 2 * tp + 1 > maxpos;
            uint32_t* col = reinterpret_cast<uint32_t*>(&vt[vc * 8][2 * tp]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t a = za ? 0u : vr[0][e], b = zb ? 0u : vr[1][e];
                col[(2 * e) * (kVtStride / 2)] = (a & 0xFFFFu) | (b << 16);
                col[(2 * e + 1) * (kVtStride / 2)] = (a >> 16) | (b & 0xFFFF0000u);
            }
        }
        // Next step's loads go out now and land while this step computes (the
        // last step reloads itself, so that no load sits under a branch).
        load_step(min(st + 1, nsteps - 1));
        lds_barrier();                          // K and V^T of the step are in LDS
        // K as the B operand: token r16 of each block, chunks g + 4c.
        u32x4 k0[NQ], k1[NQ];
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            const int cc = g + 4 * c;
            k0[c] = kl[buf][r16 * CH + (cc ^ (r16 & (CH - 1)))];
            k1[c] = kl[buf][(16 + r16) * CH + (cc ^ ((16 + r16) & (CH - 1)))];
        }
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            // logits[row 4g+j of tile t][token t0 + b*16 + r16]
            f32x4 acc0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
#pragma unroll
            for (int c = 0; c < NQ; ++c) {
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[t][c]),
                                                               __builtin_bit_cast(bf16x8, k0[c]), acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[t][c]),
                                                               __builtin_bit_cast(bf16x8, k1[c]), acc1, 0, 0, 0);
            }
            float alpha[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // Masked logits are dropped by select (they may be NaN in block tails).
                const float x0 = t0 + r16 <= pos[t][j] ? acc0[j] * p.scale_log2 : -INFINITY;
                const float x1 = t0 + 16 + r16 <= pos[t][j] ? acc1[j] * p.scale_log2 : -INFINITY;
                // Token 0 is visible to every row, so the running max is finite
                // from the first step on.
                const float mn = fmaxf(m[t][j], row_max16(fmaxf(x0, x1)));
                alpha[j] = __builtin_amdgcn_exp2f(m[t][j] - mn);
                const float p0 = __builtin_amdgcn_exp2f(x0 - mn);
                const float p1 = __builtin_amdgcn_exp2f(x1 - mn);
                lsum[t][j] = lsum[t][j] * alpha[j] + p0 + p1;
                m[t][j] = mn;
                pl[wave][16 * t + 4 * g + j][r16] = p0;
                pl[wave][16 * t + 4 * g + j][16 + r16] = p1;
            }
#pragma unroll
            for (int n = 0; n < NT; ++n)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    o[t][n][j] *= alpha[j];
        }
        // This wave's P (written and read by this wave only) is in LDS.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // P as the A operand (row r16, tokens 8g..8g+7), split into bf16 hi + lo.
        u16x8 phi[RT], plo[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            const f32x4 a0 = *reinterpret_cast<const f32x4*>(&pl[wave][16 * t + r16][8 * g]);
            const f32x4 a1 = *reinterpret_cast<const f32x4*>(&pl[wave][16 * t + r16][8 * g + 4]);
            const float pv[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            split_bf16x8(pv, phi[t], plo[t]);
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const u16x8 vb = *reinterpret_cast<const u16x8*>(&vt[n * 16 + r16][8 * g]);
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                o[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, phi[t]),
                                                                  __builtin_bit_cast(bf16x8, vb), o[t][n], 0, 0, 0);
                o[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, plo[t]),
                                                                  __builtin_bit_cast(bf16x8, vb), o[t][n], 0, 0, 0);
            }
        }
    }

    // Output rows 4g+j of each tile, columns n*16 + r16.
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float srow = row_sum16(lsum[t][j]);
            const int r = row0 + 16 * t + 4 * g + j;
            if (r >= rows)
                continue;
            const int64_t base = out_row(r) * D;
            const float inv = 1.0f / srow;
#pragma unroll
            for (int n = 0; n < NT; ++n)
                store_row_value<OUT>(p.out, base + n * 16 + r16,
                                     poisoned ? __builtin_nanf("") : o[t][n][j] * inv);
        }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int head_size, int out_bf16, int num_seqs,
                          int row_tiles, hipStream_t stream) {
    const dim3 grid(row_tiles, p.num_kv_heads, num_seqs);
    const dim3 block(kPrefillWaves * kWave);
    if (head_size == 64) {
        if (out_bf16)
            hipLaunchKernelGGL((prefill_kernel<64, BF16>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((prefill_kernel<64, F32>), grid, block, 0, stream, p);
    } else {
        if (out_bf16)
            hipLaunchKernelGGL((prefill_kernel<128, BF16>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((prefill_kernel<128, F32>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace pa

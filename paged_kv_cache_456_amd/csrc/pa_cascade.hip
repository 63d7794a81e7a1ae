// pa_cascade.hip -- attention over a prefix that every sequence shares, for
// gfx950 (CDNA4).
//
// Two requests with a common prefix can share the same physical blocks
// ("Idea 1: PagedAttention" on the day-9 post, "Why this wins"). When every
// sequence of a batch maps the same leading blocks, each KV head's prefix K
// and V are the same for all S * G query rows that read that head, so the
// prefix part of decode attention is a dense product: logits = Q K^T over
// [S * G rows] x [prefix tokens], and P V. This kernel computes it once per
// (KV head, 128-row tile, prefix chunk) on MFMA, and writes per-row partials
// (max m, sum s, normalised output o) of the chunk into the partition slots
// of the partitioned decode's workspace; the suffix of each sequence is
// decoded by the paged kernel and the log-sum-exp reduce combines both, so
// the result is the same attention as a plain decode over the whole context.
//
// Per workgroup (4 waves of two 16-row MFMA tiles each: a wave's K loads,
// the V transpose and the barriers of a step serve 32 query rows), per step
// of 32 prefix tokens (two blocks):
//   * the step's K is loaded once per workgroup into LDS (rows XOR-swizzled
//     so that reads in the MFMA B-operand layout, token = lane % 16, are free
//     of bank conflicts); Q^T K on v_mfma_f32_16x16x32_bf16 gives
//     logits[row][token];
//   * online softmax per row (running max and sum, base 2); the row max is a
//     16-lane DPP row reduction;
//   * P goes through LDS into the A-operand layout and is split into a bf16
//     high part and a bf16 remainder, so P.V keeps about 16 bits of P;
//   * V is written to LDS transposed (token-contiguous rows, padded so that
//     the B-operand reads are conflict-free) and P.V runs on MFMA with the
//     output rows in the same lanes as the softmax state;
//   * K and V^T live in two LDS buffers used on alternate steps, so one
//     barrier per step suffices.
#include "pa_device.h"

namespace pa {
namespace {

using namespace dev;

constexpr int kStepTokens = 32;                 // two blocks per step
constexpr int kVtStride = kStepTokens + 8;      // bf16 per transposed V row (80 bytes)
constexpr int kPStride = kStepTokens + 4;       // floats per P row in LDS (144 bytes)

template <int D>
__global__ __launch_bounds__(kCascadeWaves * kWave)
__attribute__((amdgpu_waves_per_eu(2)))   // 2 waves per SIMD: 247 VGPRs, no spill (D = 128)
void cascade_prefix_kernel(CascadeParams p) {
    constexpr int ROW = D * 2;                  // bytes per token row (bf16)
    constexpr int TILE = kBlockSize * ROW;
    constexpr int CH = ROW / 16;                // 16-byte chunks per row
    constexpr int NQ = CH / 4;                  // K chunks per lane per tile
    constexpr int NT = D / 16;                  // 16-column output tiles
    constexpr int VITEMS = (kStepTokens / 2) * CH;   // (token pair, chunk) items of a step
    constexpr int RT = kCascadeRowTiles;             // 16-row tiles per wave
    static_assert(VITEMS <= kCascadeWaves * kWave && (kCascadeWaves * kWave) % VITEMS == 0,
                  "one V item per thread");
    static_assert(kCascadeChunkBlocks <= kWave, "a chunk's block ids fit one per lane");

    constexpr int KITEMS = kStepTokens * CH;         // 16-byte K chunks of a step
    constexpr int KPT = KITEMS / (kCascadeWaves * kWave);   // K chunks per thread
    static_assert(KPT >= 1 && KITEMS % (kCascadeWaves * kWave) == 0, "whole K chunks per thread");
    // K and V^T of a step, two buffers each, alternating per step (a buffer is
    // written again two steps later, after a barrier every wave passes only
    // once done with it); K rows XOR-swizzled (chunk j of token t at slot
    // j ^ (t mod CH)) so that the B-operand reads hit 16 different banks.
    __shared__ __attribute__((aligned(16))) u32x4 kl[2][KITEMS];
    __shared__ __attribute__((aligned(16))) uint16_t vt2[2][D][kVtStride];
    __shared__ __attribute__((aligned(16))) float pl[kCascadeWaves][16 * RT][kPStride];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int g = lane >> 4;
    const int r16 = lane & 15;
    const int kvh = blockIdx.x;
    const int chunk = blockIdx.z;
    const int G = p.group, Hq = p.num_q_heads, Hkv = p.num_kv_heads;
    const int rows = p.num_seqs * G;
    const int row0 = blockIdx.y * (kCascadeWaves * 16 * RT) + wave * 16 * RT;

    // Query rows of this wave as the MFMA A operand: tile t, lane row r16.
    u32x4 qa[RT][NQ];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int r = row0 + 16 * t + r16;
        const bool live = r < rows;
        const int seq = live ? r / G : 0, hh = live ? r - (r / G) * G : 0;
        const char* qp = static_cast<const char*>(p.q) +
                         ((int64_t)seq * Hq + (int64_t)kvh * G + hh) * ROW;
#pragma unroll
        for (int c = 0; c < NQ; ++c)
            qa[t][c] = live ? *reinterpret_cast<const u32x4*>(qp + (g + 4 * c) * 16)
                            : u32x4{0u, 0u, 0u, 0u};
    }

    // The chunk's prefix block ids (row 0 of the tables), one per lane. An id
    // outside the pool poisons the chunk (NaN partials) and is read as block 0.
    const int cb0 = chunk * p.chunk_blocks;
    const int nblk = min(p.chunk_blocks, p.num_prefix_blocks - cb0);
    int id_l = lane < nblk ? p.block_tables[cb0 + lane] : 0;
    const bool bad_l = id_l < 0 || static_cast<int64_t>(id_l) >= p.num_blocks;
    const bool poisoned = __ballot(bad_l) != 0;
    id_l = bad_l ? 0 : id_l;
    const int nsteps = (nblk + 1) / 2;

    const char* kbase = static_cast<const char*>(p.k_cache) + (int64_t)kvh * TILE;
    const char* vbase = static_cast<const char*>(p.v_cache) + (int64_t)kvh * TILE;
    const int64_t blk_stride = (int64_t)Hkv * TILE;
    // V item of this thread: token pair tp (tokens 2tp, 2tp + 1 of the step), chunk vc.
    const int vi = threadIdx.x % VITEMS;
    const int tp = vi % (kStepTokens / 2), vc = vi / (kStepTokens / 2);
    const int vblk = tp >> 3;                   // which block of the step
    const int voff = (2 * tp - 16 * vblk) * ROW + vc * 16;

    // K chunks of this thread: item q = threadIdx.x + k * threads is chunk
    // q % CH of token q / CH of the step (block (q / CH) / 16), stored at its
    // swizzled slot.
    int kslot[KPT], koff[KPT], kblk[KPT];
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
        const int q = threadIdx.x + k * kCascadeWaves * kWave;
        const int t = q / CH, j = q % CH;
        kslot[k] = t * CH + (j ^ (t & (CH - 1)));
        kblk[k] = t >> 4;
        koff[k] = (t & 15) * ROW + j * 16;
    }
    // Loads of step st: this thread's K chunks of its two blocks (a lone last
    // block is read twice and masked) and its V pair.
    u32x4 kq[KPT], vr[2];
    auto load_step = [&](int st) {
        const int b0 = 2 * st, b1 = min(2 * st + 1, nblk - 1);
        const int id0 = __builtin_amdgcn_readlane(id_l, b0);
        const int id1 = __builtin_amdgcn_readlane(id_l, b1);
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
        const bool pair = 2 * st + 1 < nblk;
        const int buf = st & 1;
        auto& vt = vt2[buf];
        // K of the step into LDS; V transposed into LDS (two adjacent tokens
        // per 32-bit word).
#pragma unroll
        for (int k = 0; k < KPT; ++k)
            kl[buf][kslot[k]] = kq[k];
        {
            uint32_t* col = reinterpret_cast<uint32_t*>(&vt[vc * 8][2 * tp]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t a = vr[0][e], b = vr[1][e];
                col[(2 * e) * (kVtStride / 2)] = (a & 0xFFFFu) | (b << 16);
                col[(2 * e + 1) * (kVtStride / 2)] = (a >> 16) | (b & 0xFFFF0000u);
            }
        }
        // Next step's loads go out now and land while this step computes (the
        // last step reloads itself, so that no load sits under a branch).
        load_step(min(st + 1, nsteps - 1));
        lds_barrier();                     // K and V^T of the step are in LDS
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
            // logits[row 4g+j of tile t][token b*16 + r16]
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
                const float x0 = acc0[j] * p.scale_log2;
                const float x1 = pair ? acc1[j] * p.scale_log2 : -INFINITY;
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

    // Row partials of this chunk: rows 4g+j of each tile, columns n*16 + r16.
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float srow = row_sum16(lsum[t][j]);
            const int r = row0 + 16 * t + 4 * g + j;
            if (r >= rows)
                continue;
            const int seq = r / G, hh = r - (r / G) * G;
            const int64_t pi = ((int64_t)seq * Hq + (int64_t)kvh * G + hh) * p.part_stride +
                               p.slot_base + chunk;
            const float inv = 1.0f / srow;
#pragma unroll
            for (int n = 0; n < NT; ++n)
                p.part_out[pi * D + n * 16 + r16] = poisoned ? __builtin_nanf("") : o[t][n][j] * inv;
            if (r16 == 0) {
                p.part_max[pi] = poisoned ? 0.0f : m[t][j] * kLn2;
                p.part_sum[pi] = poisoned ? __builtin_nanf("") : srow;
            }
        }
}

}  // namespace

hipError_t launch_cascade_prefix(const CascadeParams& p, int head_size, int num_chunks,
                                 hipStream_t stream) {
    const int rows = p.num_seqs * p.group;
    constexpr int kTileRows = kCascadeWaves * 16 * kCascadeRowTiles;
    const dim3 grid(p.num_kv_heads, (rows + kTileRows - 1) / kTileRows, num_chunks);
    if (head_size == 64)
        hipLaunchKernelGGL(cascade_prefix_kernel<64>, grid, dim3(kCascadeWaves * kWave), 0, stream, p);
    else
        hipLaunchKernelGGL(cascade_prefix_kernel<128>, grid, dim3(kCascadeWaves * kWave), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa

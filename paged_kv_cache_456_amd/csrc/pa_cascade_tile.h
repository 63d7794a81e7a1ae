// pa_cascade_tile.h -- one tile of the shared-prefix product: the query rows
// of one 64-row tile of one KV head against one chunk of the prefix, on the
// MFMA step of pa_tile.h, written as per-row partials (max m, sum s,
// normalised output o) to the chunk's slot of the partitioned workspace.
// Used by the standalone shared-prefix kernel (pa_cascade.hip) and by the
// shared launch in which some workgroups take prefix tiles while the others
// decode the suffixes (pa_decode.hip). The caller provides the step's LDS
// and calls it with all kCascadeWaves waves of the workgroup.
#pragma once

#include "pa_tile.h"

namespace pa {
namespace tile {

static_assert(sizeof(Lds<64, kCascadeWaves>) == cascade_tile_lds_bytes(64) &&
                  sizeof(Lds<128, kCascadeWaves>) == cascade_tile_lds_bytes(128),
              "the host's size of the tile LDS");

template <int D>
__device__ __forceinline__ void prefix_tile(const CascadeParams& p, Lds<D, kCascadeWaves>& lds, int kvh,
                                            int row_tile, int chunk) {
    using S = Shape<D, kCascadeWaves>;
    constexpr int ROW = S::ROW, NQ = S::NQ, NT = S::NT, RT = kCascadeRowTiles;
    static_assert(kCascadeChunkBlocks <= kWave && kCascadeSharedChunkBlocks <= kWave &&
                      kCascadeSharedChunkBlocks >= kCascadeChunkBlocks,
                  "a chunk's block ids fit one per lane; the longer chunks need no more slots");

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int g = lane >> 4;
    const int r16 = lane & 15;
    const int G = p.group, Hq = p.num_q_heads, Hkv = p.num_kv_heads;
    const int rows = p.num_seqs * G;
    const int row0 = row_tile * kCascadeTileRows + wave * 16 * RT;

    // Query rows of this wave as the MFMA B operand: tile t, lane row r16.
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

    const char* kbase = static_cast<const char*>(p.k_cache) + (int64_t)kvh * S::TILE;
    const char* vbase = static_cast<const char*>(p.v_cache) + (int64_t)kvh * S::TILE;
    const int64_t blk_stride = (int64_t)Hkv * S::TILE;
    Loader<D, kCascadeWaves> ld;
    ld.init();
    RowState<D, RT> rs;
    rs.reset();
    // A lone last block is read twice; its second copy is hidden.
    run_steps<D, kCascadeWaves>(
        nsteps,
        [&](StepData<D, kCascadeWaves>& d, int st) {
            ld.load(d, kbase, vbase, blk_stride, __builtin_amdgcn_readlane(id_l, 2 * st),
                    __builtin_amdgcn_readlane(id_l, min(2 * st + 1, nblk - 1)));
        },
        [&](const StepData<D, kCascadeWaves>& d, int, int buf) {
            ld.stage(d, lds, buf, kStepTokens);
        },
        [&](int st, int buf) {
            const bool pair = 2 * st + 1 < nblk;
            attend<D, kCascadeWaves, RT>(lds, buf, qa, p.scale_log2,
                                               [&](int, int tok) { return pair || tok < kBlockSize; },
                                               [&](int) { return pair; }, rs);
        });

    // Row partials of this chunk: row r16 of each tile, columns 16n + 4g + j.
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const float srow = rs.row_sum(t);
        const int r = row0 + 16 * t + r16;
        if (r >= rows)
            continue;
        const int seq = r / G, hh = r - (r / G) * G;
        const int64_t pi = ((int64_t)seq * Hq + (int64_t)kvh * G + hh) * p.part_stride +
                           p.slot_base + chunk;
        const float inv = 1.0f / srow;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const f32x4 v = poisoned ? f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                                             __builtin_nanf("")}
                                     : rs.o[t][n] * inv;
            *reinterpret_cast<f32x4*>(p.part_out + pi * D + n * 16 + 4 * g) = v;
        }
        if (g == 0) {
            p.part_max[pi] = poisoned ? 0.0f : rs.m[t] * dev::kLn2;
            p.part_sum[pi] = poisoned ? __builtin_nanf("") : srow;
        }
    }
}

}  // namespace tile
}  // namespace pa

// pa_cascade.hip -- attention over a prefix that every sequence shares, for
// gfx950 (CDNA4).
//
// Two requests with a common prefix can share the same physical blocks
// ("Idea 1: PagedAttention" on the day-9 post, "Why this wins"). When every
// sequence of a batch maps the same leading blocks, each KV head's prefix K
// and V are the same for all S * G query rows that read that head, so the
// prefix part of decode attention is a dense product: logits = Q K^T over
// [S * G rows] x [prefix tokens], and P V. This kernel computes it once per
// (KV head, 64-row tile, prefix chunk) on MFMA, and writes per-row partials
// (max m, sum s, normalised output o) of the chunk into the partition slots
// of the partitioned decode's workspace; the suffix of each sequence is
// decoded by the paged kernel and the log-sum-exp reduce combines both, so
// the result is the same attention as a plain decode over the whole context.
//
// Per workgroup: 4 waves of one 16-row MFMA tile each, over a chunk of 32
// prefix blocks (a chunk's partials are written once per row, so longer
// chunks write fewer of them; the combine reads fewer back), one step of 32
// prefix tokens (two blocks) at a time, the step of
// pa_tile.h: K and V^T staged in LDS (two buffers, one barrier per step),
// K Q^T and V^T P^T on v_mfma_f32_16x16x32_bf16 with P kept in registers
// (split into a bf16 high part and remainder), online softmax per row with
// its statistics in the row's four lanes. The next step's K and V are
// requested before this step computes.
#include "pa_tile.h"

namespace pa {
namespace {

using namespace dev;

template <int D>
__global__ __launch_bounds__(kCascadeWaves * kWave)
__attribute__((amdgpu_waves_per_eu(2)))
void cascade_prefix_kernel(CascadeParams p) {
    using S = tile::Shape<D, kCascadeWaves>;
    constexpr int ROW = S::ROW, NQ = S::NQ, NT = S::NT, RT = kCascadeRowTiles;
    static_assert(kCascadeChunkBlocks <= kWave, "a chunk's block ids fit one per lane");
    __shared__ __attribute__((aligned(16))) tile::Lds<D, kCascadeWaves> lds;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int g = lane >> 4;
    const int r16 = lane & 15;
    const int kvh = blockIdx.x;
    const int chunk = blockIdx.z;
    const int G = p.group, Hq = p.num_q_heads, Hkv = p.num_kv_heads;
    const int rows = p.num_seqs * G;
    const int row0 = blockIdx.y * (kCascadeWaves * 16 * RT) + wave * 16 * RT;

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
    tile::Loader<D, kCascadeWaves> ld;
    ld.init();
    tile::RowState<D, RT> rs;
    rs.reset();
    // A lone last block is read twice; its second copy is hidden.
    tile::run_steps<D, kCascadeWaves>(
        nsteps,
        [&](tile::StepData<D, kCascadeWaves>& d, int st) {
            ld.load(d, kbase, vbase, blk_stride, __builtin_amdgcn_readlane(id_l, 2 * st),
                    __builtin_amdgcn_readlane(id_l, min(2 * st + 1, nblk - 1)));
        },
        [&](const tile::StepData<D, kCascadeWaves>& d, int, int buf) {
            ld.stage(d, lds, buf, tile::kStepTokens);
        },
        [&](int st, int buf) {
            const bool pair = 2 * st + 1 < nblk;
            tile::attend<D, kCascadeWaves, RT>(lds, buf, qa, p.scale_log2,
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
            p.part_max[pi] = poisoned ? 0.0f : rs.m[t] * kLn2;
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

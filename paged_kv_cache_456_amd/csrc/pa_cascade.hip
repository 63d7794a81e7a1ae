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
#include "pa_cascade_tile.h"

namespace pa {
namespace {

template <int D>
__global__ __launch_bounds__(kCascadeWaves * kWave)
__attribute__((amdgpu_waves_per_eu(2)))
void cascade_prefix_kernel(CascadeParams p) {
    __shared__ __attribute__((aligned(16))) tile::Lds<D, kCascadeWaves> lds;
    tile::prefix_tile<D>(p, lds, blockIdx.x, blockIdx.y, blockIdx.z);
}

}  // namespace

hipError_t launch_cascade_prefix(const CascadeParams& p, int head_size, hipStream_t stream) {
    const dim3 grid(p.num_kv_heads, p.row_tiles, p.num_chunks);
    if (head_size == 64)
        hipLaunchKernelGGL(cascade_prefix_kernel<64>, grid, dim3(kCascadeWaves * kWave), 0, stream, p);
    else
        hipLaunchKernelGGL(cascade_prefix_kernel<128>, grid, dim3(kCascadeWaves * kWave), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa

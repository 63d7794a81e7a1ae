// pa_stream.hip -- the streaming-read calibration kernel for gfx950.
//
// Decode attention is bounded by the rate at which HBM delivers the KV tiles,
// so the rate a plain read reaches on this GPU is the practical ceiling its
// kernels are measured against (next to the nominal 8 TB/s). This kernel reads
// every 16-byte word of a buffer once, with the same nontemporal 16-byte loads
// the decode kernels use for K and V, eight loads in flight per thread, and
// folds the words with XOR so that no load can be dropped: wave w writes the
// XOR of the words it read to sink[w]. The XOR of all sink words is the XOR of
// all words of the buffer, whatever the grid.
#include "pa_internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4* src, int64_t n,
                                                                    u32x4* sink) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kStreamThreads;
    int64_t i = static_cast<int64_t>(blockIdx.x) * kStreamThreads + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (kStreamUnroll - 1) * stride < n; i += kStreamUnroll * stride) {
        u32x4 v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u)
            v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u)
            acc ^= v[u];
    }
    for (; i < n; i += stride)
        acc ^= __builtin_nontemporal_load(src + i);
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            acc[c] ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc[c]), off, kWave));
    if ((threadIdx.x & (kWave - 1)) == 0)
        sink[static_cast<int64_t>(blockIdx.x) * (kStreamThreads / kWave) + threadIdx.x / kWave] = acc;
}

}  // namespace

int stream_read_waves_per_workgroup() { return kStreamThreads / kWave; }

hipError_t launch_stream_read(const void* src, int64_t num_words, void* sink, int num_workgroups,
                              hipStream_t stream) {
    hipLaunchKernelGGL(stream_read_kernel, dim3(num_workgroups), dim3(kStreamThreads), 0, stream,
                       static_cast<const u32x4*>(src), num_words, static_cast<u32x4*>(sink));
    return hipGetLastError();
}

}  // namespace pa

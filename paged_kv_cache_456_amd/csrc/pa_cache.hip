// pa_cache.hip -- the KV-cache write (reshape_and_cache) for gfx950.
//
// Each new token's key and value vectors go into the slot the host chose for
// it: row slot % 16 of physical block slot / 16, for every KV head. The pages
// say a request keeps the key/value state of each token it produced and holds
// only the blocks those tokens fill ("The problem a naive server has" and
// "The idea vLLM started from: pages" on "What vLLM Is and Why It Exists");
// the slot numbering is this library's convention.
//
// The copy is a bit copy in 16-byte pieces: one workgroup per token, its
// threads walking the token's Hkv * D elements of K, then of V. Source reads
// are contiguous; each head's destination row is contiguous.
#include "pa_internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCacheThreads = 256;

__global__ __launch_bounds__(kCacheThreads) void reshape_and_cache_kernel(CacheParams p) {
    const int64_t t = blockIdx.x;
    const int cph = p.row_bytes / 16;              // 16-byte pieces per head row
    const int chunks = p.num_kv_heads * cph;       // pieces per token per tensor
    // The slot is needed only for the stores: its load and the source loads
    // are in flight together.
    const int64_t slot = p.slot_mapping[t];
    for (int c = threadIdx.x; c < 2 * chunks; c += blockDim.x) {
        const bool is_v = c >= chunks;
        const int cc = is_v ? c - chunks : c;
        const u32x4 piece = *reinterpret_cast<const u32x4*>((is_v ? p.value : p.key) + (t * chunks + cc) * 16);
        if (slot < 0 || slot >= p.num_slots)   // padding token, or a slot outside the pool
            return;
        const int64_t blk = slot / kBlockSize;
        const int64_t off = slot % kBlockSize;
        const int h = cc / cph;
        const int w = cc - h * cph;
        uint8_t* dst = (is_v ? p.value_cache : p.key_cache) +
                       ((blk * p.num_kv_heads + h) * kBlockSize + off) * p.row_bytes + w * 16;
        *reinterpret_cast<u32x4*>(dst) = piece;
    }
}

// Copy-on-write block copy ("Idea 1: PagedAttention" on the day-9 post: when
// a shared block must diverge, only that block is copied). Each pair
// (src, dst) copies physical block src of both pools onto block dst. Grid:
// (pairs, 2 pools); a workgroup streams one block of one pool
// (Hkv * 16 * D * elem bytes) in 16-byte pieces, kCopyUnroll pieces in flight
// per thread, past the caches (nothing reads the copy in this kernel).
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 8;

// One block of one pool, `block_bytes` bytes, copied by the workgroup.
__device__ __forceinline__ void copy_block(const uint8_t* src, uint8_t* dst, int64_t block_bytes) {
    const u32x4* from = reinterpret_cast<const u32x4*>(src);
    u32x4* to = reinterpret_cast<u32x4*>(dst);
    const int64_t n = block_bytes / 16;
    for (int64_t c0 = threadIdx.x; c0 < n; c0 += static_cast<int64_t>(blockDim.x) * kCopyUnroll) {
        u32x4 v[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const int64_t c = c0 + static_cast<int64_t>(u) * blockDim.x;
            if (c < n)
                v[u] = __builtin_nontemporal_load(from + c);
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const int64_t c = c0 + static_cast<int64_t>(u) * blockDim.x;
            if (c < n)
                __builtin_nontemporal_store(v[u], to + c);
        }
    }
}

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyParams p) {
    const int64_t i = blockIdx.x;
    const int64_t src = p.block_mapping[2 * i];
    const int64_t dst = p.block_mapping[2 * i + 1];
    if (src < 0 || dst < 0 || src >= p.num_blocks || dst >= p.num_blocks)
        return;                                    // skipped pair, or an id outside the pool
    uint8_t* pool = blockIdx.y ? p.value_cache : p.key_cache;
    copy_block(pool + src * p.block_bytes, pool + dst * p.block_bytes, p.block_bytes);
}

// Swap of whole blocks between two pairs of pools (preemption moves a
// request's blocks out of the GPU pools and back: "Why read its source at
// all" on "What vLLM Is and Why It Exists"). Pair i copies block src of the
// source pools onto block dst of the destination pools; one side is usually
// pinned host memory, read or written by the kernel across the host link.
// Grid: (pairs, 2 pools), as the copy above.
__global__ __launch_bounds__(kCopyThreads) void swap_blocks_kernel(SwapParams p) {
    const int64_t i = blockIdx.x;
    const int64_t src = p.block_mapping[2 * i];
    const int64_t dst = p.block_mapping[2 * i + 1];
    if (src < 0 || dst < 0 || src >= p.src_num_blocks || dst >= p.dst_num_blocks)
        return;                                    // skipped pair, or an id outside its pool
    const uint8_t* from = blockIdx.y ? p.src_value : p.src_key;
    uint8_t* to = blockIdx.y ? p.dst_value : p.dst_key;
    copy_block(from + src * p.block_bytes, to + dst * p.block_bytes, p.block_bytes);
}

}  // namespace

hipError_t launch_copy_blocks(const CopyParams& p, int64_t num_pairs, hipStream_t stream) {
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<unsigned>(num_pairs), 2),
                       dim3(kCopyThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_swap_blocks(const SwapParams& p, int64_t num_pairs, hipStream_t stream) {
    hipLaunchKernelGGL(swap_blocks_kernel, dim3(static_cast<unsigned>(num_pairs), 2),
                       dim3(kCopyThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_cache(const CacheParams& p, int64_t num_tokens, hipStream_t stream) {
    const int pieces = 2 * p.num_kv_heads * (p.row_bytes / 16);
    int threads = ((pieces + kWave - 1) / kWave) * kWave;
    if (threads > kCacheThreads)
        threads = kCacheThreads;
    hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(static_cast<unsigned>(num_tokens)),
                       dim3(threads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa

// pa_internal.h -- types shared by the HIP kernels and the C-ABI layer of the
// paged decode attention library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlockSize = 16;   // tokens per KV block
constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kMaxWaves = 8;     // waves per decode workgroup (single pass)
constexpr int kPartWaves = 4;    // waves per decode workgroup (partitioned)
constexpr int kReduceThreads = 256;
constexpr int kReduceMaxWaves = 16;      // partition combine: one wave per query head of a group
constexpr int kCascadeWaves = 4;          // waves per prefix workgroup
constexpr int kCascadeRowTiles = 1;       // 16-row tiles per wave (64 query rows per workgroup)
constexpr int kCascadeChunkBlocks = 32;   // prefix blocks per prefix workgroup (sizes the workspace)
constexpr int kCascadeSharedChunkBlocks = 64;   // prefix blocks per tile in the shared launch
constexpr int kCascadeTileRows = kCascadeWaves * 16 * kCascadeRowTiles;   // query rows per prefix tile
constexpr int kPrefillWaves = 4;          // waves per multi-token-query workgroup
constexpr int kPrefillRowTiles = 2;       // 16-row tiles per wave (128 rows per workgroup)

// Element tags for the KV dtype.
struct BF16 {
    static constexpr int kBytes = 2;
};
struct F32 {
    static constexpr int kBytes = 4;
};

// Kernel arguments of the decode kernel (one struct, passed by value).
struct DecodeParams {
    const void* q;                 // [S][Hq][D]
    const void* k_cache;           // [NB][Hkv][16][D]
    const void* v_cache;           // [NB][Hkv][16][D]
    const int32_t* block_tables;   // [S][MB]
    const int32_t* context_lens;   // [S]
    void* out;                     // [S][Hq][D]
    float* part_max;               // [S][Hq][NP]  (partitioned) or nullptr
    float* part_sum;               // [S][Hq][NP]
    float* part_out;               // [S][Hq][NP][D]
    int64_t num_blocks;
    int max_blocks_per_seq;
    int num_q_heads;
    int num_kv_heads;
    int group;                     // Hq / Hkv
    int partition_blocks;          // blocks per partition (single pass: >= MB)
    int num_partitions;            // partitions a context may span (longer ones are unreadable)
    int part_stride;               // partial slots per row in the workspace (>= num_partitions)
    int num_seqs;
    int persistent;                // 1: persistent schedule (resident grid), 0: one workgroup per partition
    int skip_blocks;               // leading table entries that are not part of this call
    int table_blocks;              // max_blocks_per_seq - skip_blocks
    int partials_only;             // 1: write partials for every partition, never `out`
    float scale_log2;              // scale * log2(e)
    const void* new_key;           // [S][Hkv][D]: each sequence's new token, stored at position
    const void* new_value;         //   L - 1 and attended from here (nullptr: no write)
};

struct ReduceParams {
    const int32_t* context_lens;
    const float* part_max;         // [S][Hq][part_stride], natural-log units
    const float* part_sum;         // [S][Hq][part_stride]
    const float* part_out;         // [S][Hq][part_stride][D]
    void* out;                     // [S][Hq][D]
    int64_t num_blocks;
    int max_blocks_per_seq;
    int num_q_heads;
    int num_kv_heads;
    int group;
    int num_partitions;            // as in DecodeParams
    int part_stride;
    int partition_blocks;
    int skip_blocks;
    int table_blocks;
    int extra_base;                // shared-prefix partials sit in slots [extra_base,
    int extra_count;               //   extra_base + extra_count) of every row (cascade)
};

struct CacheParams {
    const uint8_t* key;
    const uint8_t* value;
    uint8_t* key_cache;
    uint8_t* value_cache;
    const int64_t* slot_mapping;
    int64_t num_slots;             // NB * 16
    int num_kv_heads;
    int row_bytes;                 // D * element bytes
};

// Query heads per KV head that a decode kernel instance is compiled for:
// the group size rounded up to 1, 2, 4, 8 or 16.
constexpr int decode_gmax(int group) {
    return group <= 1 ? 1 : group <= 2 ? 2 : group <= 4 ? 4 : group <= 8 ? 8 : 16;
}

// Blocks each wave loads per round. One: the next round's K and V tiles are
// requested while a round computes, so a wave keeps one to two blocks (8-16
// KB for bf16 D = 128) in flight; measured on MI355X, more requests in flight
// per wave (two blocks per round) saturate the L1 address translation's
// in-flight tracking and run slower.
constexpr int decode_bpw(int /*elem_bytes*/, int /*head_size*/, int /*gmax*/) { return 1; }

// Row stride, in floats, of the per-wave softmax-weight tile in LDS.
constexpr int decode_pstride(int gmax) { return gmax < 4 ? 4 : gmax; }

// Floats of decode LDS per workgroup of `waves` waves (layout below).
constexpr size_t decode_lds_floats(int elem_bytes, int head_size, int group, int waves) {
    return static_cast<size_t>(waves) *
           (static_cast<size_t>(decode_bpw(elem_bytes, head_size, decode_gmax(group))) * 16 *
                decode_pstride(decode_gmax(group)) +
            2 * decode_pstride(decode_gmax(group)) +
            static_cast<size_t>(decode_gmax(group)) * head_size);
}

// Dynamic LDS bytes of a decode workgroup of `waves` waves:
//   p    [waves][bpw * 16][pstride]  softmax weights of the current round
//   m, s [waves][pstride]            per-wave running max and sum
//   o    [waves][gmax][D]            per-wave unnormalised output
constexpr size_t decode_lds_bytes(int elem_bytes, int head_size, int group, int waves) {
    return sizeof(float) * decode_lds_floats(elem_bytes, head_size, group, waves);
}

// Persistent schedule: the largest batch (context lengths and their prefix
// sums are kept in LDS); up to kMaxSortedSeqs sequences the items are ordered
// by size class (kSizeClasses classes of partly filled last partitions).
constexpr int kMaxPersistentSeqs = 4096;
constexpr int kMaxSortedSeqs = 1024;
constexpr int kSizeClasses = 4;

// LDS bytes of the shared-prefix tile step for head size D (K and V^T, two
// buffers each): 2 * 32 tokens * 2D bytes of K plus 2 * D rows * 40 bf16 of V^T.
constexpr size_t cascade_tile_lds_bytes(int head_size) {
    return static_cast<size_t>(288) * head_size;
}

// The shared launch of a shared-prefix batch (some workgroups take prefix
// tiles, the others decode suffixes): LDS floats before the suffixes'
// context lengths and partition prefix sums, enough for either kind of work
// (bf16 KV, kPartWaves waves).
constexpr size_t cascade_shared_area_floats(int head_size, int group) {
    return decode_lds_floats(2, head_size, group, kPartWaves) > cascade_tile_lds_bytes(head_size) / 4
               ? decode_lds_floats(2, head_size, group, kPartWaves)
               : cascade_tile_lds_bytes(head_size) / 4;
}

// Extra LDS of the persistent schedule: lens [S], the inclusive prefix sums
// ([1 + kSizeClasses][S] when the items are ordered by size class, else [S])
// and 1 + kSizeClasses totals.
constexpr size_t persistent_lds_bytes(int num_seqs) {
    return sizeof(int) * ((num_seqs <= kMaxSortedSeqs ? 2 + kSizeClasses : 2) * static_cast<size_t>(num_seqs) +
                          1 + kSizeClasses);
}

// Work-balanced decode (pa_decode_balanced.hip): the (sequence, KV head,
// block) units of the batch cut into equal contiguous ranges, one per
// resident workgroup and, within it, one per wave.
constexpr int kBalancedWaves = 4;               // waves per workgroup
constexpr int kMaxBalancedWorkgroups = 1024;    // grid cap; sizes the workspace
constexpr int kMaxBalancedSeqs = 4096;          // first units of all sequences sit in LDS

struct BalancedParams {
    DecodeParams d;                // part_max / part_sum: [2 * wgs][group] (max in base 2),
                                   // part_out: [2 * wgs][group][D]
    int4* desc;                    // [wgs]: row cut at the end of a workgroup's range, its slot
                                   // there, and the last workgroup holding it; x < 0 for none
    const void* new_key;           // [S][Hkv][D]: the step's new token, written at L - 1, or nullptr
    const void* new_value;
};

// Shared-prefix (cascade) attention over the blocks every sequence shares.
struct CascadeParams {
    const void* q;                 // [S][Hq][D] bf16
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;   // the prefix ids are row 0's first num_prefix_blocks entries
    float* part_max;               // workspace partials, row stride part_stride
    float* part_sum;
    float* part_out;
    int64_t num_blocks;
    int num_prefix_blocks;
    int chunk_blocks;              // prefix blocks per workgroup
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int group;
    int part_stride;               // row stride of the partials
    int slot_base;                 // slot of prefix chunk 0
    int row_tiles;                 // 64-row tiles of the S * G query rows of a KV head
    int num_chunks;                // prefix chunks
    float scale_log2;
};


// Multi-token queries over the paged cache (prompt / chunked prefill).
struct PrefillParams {
    const void* q;                 // [T][Hq][D] bf16, T = query_start[S]
    const void* k_cache;           // [NB][Hkv][16][D] bf16
    const void* v_cache;
    const int32_t* block_tables;   // [S][MB]
    const int32_t* context_lens;   // [S]
    const int32_t* query_start;    // [S + 1]
    int64_t num_query_rows;        // T: rows of q and out
    void* out;                     // [T][Hq][D]
    int64_t num_blocks;
    int max_blocks_per_seq;
    int num_q_heads;
    int num_kv_heads;
    int group;
    int max_query_len;             // rows past this many per sequence are not computed
    float scale_log2;              // scale * log2(e)
    int row_tiles;                 // 128-row tiles per (sequence, KV head)
    int* order;                    // [S * row_tiles]: (sequence, tile) pairs, most steps first
};

constexpr int kPrefillOrderBins = 4096;   // step counts the ordering tells apart

struct CopyParams {
    uint8_t* key_cache;
    uint8_t* value_cache;
    const int64_t* block_mapping;  // [N][2]: source block, destination block
    int64_t num_blocks;
    int64_t block_bytes;           // Hkv * 16 * D * element bytes
};

struct SwapParams {
    const uint8_t* src_key;        // source pools [src_num_blocks][Hkv][16][D]
    const uint8_t* src_value;
    uint8_t* dst_key;              // destination pools [dst_num_blocks][Hkv][16][D]
    uint8_t* dst_value;
    const int64_t* block_mapping;  // [N][2]: source block, destination block
    int64_t src_num_blocks;
    int64_t dst_num_blocks;
    int64_t block_bytes;           // Hkv * 16 * D * element bytes
};

// Facts of the current device, queried once per device (pa_device_cache.cpp).
struct DeviceInfo {
    int cus;         // compute units
    int max_lds;     // LDS bytes one workgroup may use
};
hipError_t current_device_info(int* device, DeviceInfo* info);
// Workgroups of `kernel` (`threads` threads, `lds` bytes of dynamic LDS) that
// one compute unit of `device` keeps resident, queried once per combination.
hipError_t resident_workgroups_per_cu(int device, const void* kernel, int threads, size_t lds,
                                      int* per_cu);

// Launchers (pa_decode.hip, pa_cache.hip). kv: 0 = fp32, 1 = bf16.
hipError_t launch_decode(const DecodeParams& p, int kv_bf16, int head_size, int out_bf16,
                         int num_seqs, int grid_partitions, int waves, hipStream_t stream);
hipError_t launch_reduce(const ReduceParams& p, int head_size, int out_bf16, int num_seqs,
                         hipStream_t stream);
// The balanced decode and its combining kernel; max_workgroups caps the grid
// below the resident count (small batches).
hipError_t launch_decode_balanced(const BalancedParams& p, int kv_bf16, int head_size, int out_bf16,
                                  int max_workgroups, hipStream_t stream);
size_t balanced_lds_bytes_for(int kv_bf16, int head_size, int group, int num_seqs);
hipError_t launch_cache(const CacheParams& p, int64_t num_tokens, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyParams& p, int64_t num_pairs, hipStream_t stream);
hipError_t launch_swap_blocks(const SwapParams& p, int64_t num_pairs, hipStream_t stream);
// One launch for the prefix tiles and the suffixes of a shared-prefix batch
// (bf16 KV, kPartWaves-wave decode workgroups); *launched is false, and
// nothing is launched, when its LDS does not fit a workgroup.
hipError_t launch_cascade_shared(const DecodeParams& p, const CascadeParams& c, int head_size,
                                 int out_bf16, int num_seqs, int grid_partitions, bool* launched,
                                 hipStream_t stream);
hipError_t launch_cascade_prefix(const CascadeParams& p, int head_size, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, int head_size, int out_bf16, int num_seqs,
                          int row_tiles, hipStream_t stream);
int stream_read_waves_per_workgroup();
hipError_t launch_stream_read(const void* src, int64_t num_words, void* sink, int num_workgroups,
                              hipStream_t stream);

}  // namespace pa

// pa_internal.h -- types shared by the HIP kernels and the C-ABI layer of the
// paged decode attention library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlockSize = 16;   // tokens per KV block
constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kMaxWaves = 8;     // waves per decode workgroup

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
    void* out;                     // [S][Hq][D]   (single pass) or nullptr
    float* part_max;               // [S][Hq][NP]  (partitioned) or nullptr
    float* part_sum;               // [S][Hq][NP]
    float* part_out;               // [S][Hq][NP][D]
    int64_t num_blocks;
    int max_blocks_per_seq;
    int num_q_heads;
    int num_kv_heads;
    int group;                     // Hq / Hkv
    int partition_blocks;          // blocks per partition (single pass: >= MB)
    int num_partitions;            // NP, the workspace stride
    float scale_log2;              // scale * log2(e)
};

struct ReduceParams {
    const int32_t* context_lens;
    const float* part_max;
    const float* part_sum;
    const float* part_out;
    void* out;
    int num_q_heads;
    int num_partitions;
    int partition_size;
    int max_blocks_per_seq;
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

// Launchers (pa_decode.hip, pa_cache.hip). kv: 0 = fp32, 1 = bf16.
hipError_t launch_decode(const DecodeParams& p, int kv_bf16, int head_size, int out_bf16,
                         int num_seqs, int grid_partitions, int waves, hipStream_t stream);
hipError_t launch_reduce(const ReduceParams& p, int head_size, int out_bf16, int num_seqs,
                         hipStream_t stream);
hipError_t launch_cache(const CacheParams& p, int64_t num_tokens, hipStream_t stream);

// Dynamic LDS bytes of a decode workgroup.
size_t decode_lds_bytes_for(int head_size, int group, int waves);

}  // namespace pa

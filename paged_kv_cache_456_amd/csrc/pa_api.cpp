// pa_api.cpp -- the C-ABI of the paged decode attention library: argument
// checks on the host, launch geometry, and the calls into the HIP kernels.
// Every check runs before anything is enqueued; nothing here allocates,
// synchronises or keeps state.
#include <math.h>
#include <stdint.h>

#include "pa.h"
#include "pa_internal.h"

namespace {

constexpr int kMaxGroup = 16;          // query heads per KV head handled by one wave
constexpr int kMaxGridYZ = 65535;      // grid y (sequences) and z (partitions) limits
constexpr size_t kMaxDecodeLds = 64 * 1024;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool dtype_ok(pa_dtype_t t) { return t == PA_F32 || t == PA_BF16; }

int elem_bytes(pa_dtype_t t) { return t == PA_BF16 ? 2 : 4; }

size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

pa_status_t from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_EHIP; }

// Checks shared by both decode entry points. Returns PA_OK when the call may
// go ahead (num_seqs may still be 0).
pa_status_t check_decode(const void* out, pa_dtype_t out_dtype, const void* query,
                         const void* key_cache, const void* value_cache, pa_dtype_t kv_dtype,
                         const int32_t* block_tables, int max_blocks_per_seq,
                         const int32_t* context_lens, int num_seqs, int num_q_heads,
                         int num_kv_heads, int head_size, int block_size, int64_t num_blocks,
                         float scale) {
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 ||
        block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks < 0)
        return PA_EINVAL;
    if (num_q_heads % num_kv_heads != 0)
        return PA_EINVAL;
    if (!isfinite(scale))
        return PA_EINVAL;
    if (!dtype_ok(kv_dtype) || !dtype_ok(out_dtype))
        return PA_EUNSUPPORTED;
    if (block_size != pa::kBlockSize || (head_size != 64 && head_size != 128))
        return PA_EUNSUPPORTED;
    if (num_q_heads / num_kv_heads > kMaxGroup || num_seqs > kMaxGridYZ)
        return PA_EUNSUPPORTED;
    if (num_seqs == 0)
        return PA_OK;
    if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
        return PA_EINVAL;
    if (!aligned(out, 16) || !aligned(query, 16) || !aligned(key_cache, 16) ||
        !aligned(value_cache, 16) || !aligned(block_tables, 4) || !aligned(context_lens, 4))
        return PA_EINVAL;
    // Byte offsets into the pools are 64-bit; make sure they cannot overflow.
    const int64_t block_bytes = static_cast<int64_t>(num_kv_heads) * pa::kBlockSize * head_size *
                                elem_bytes(kv_dtype);
    if (num_blocks > INT64_MAX / block_bytes)
        return PA_EINVAL;
    return PA_OK;
}

pa::DecodeParams make_params(const void* query, const void* key_cache, const void* value_cache,
                             const int32_t* block_tables, int max_blocks_per_seq,
                             const int32_t* context_lens, int num_q_heads, int num_kv_heads,
                             int64_t num_blocks, float scale) {
    pa::DecodeParams p{};
    p.q = query;
    p.k_cache = key_cache;
    p.v_cache = value_cache;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.num_blocks = num_blocks;
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.group = num_q_heads / num_kv_heads;
    p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
    return p;
}

// Waves per workgroup: enough for one round to cover the blocks a workgroup
// owns (each wave takes decode_bpw blocks per round), capped by `max_waves`
// and by LDS. Partitioned launches use small (4-wave) workgroups so that two
// or more fit on a CU; the single pass uses up to 8 waves per sequence.
int choose_waves(int blocks_per_workgroup, int kv_bytes, int head_size, int group, int max_waves) {
    const int bpw = pa::decode_bpw(kv_bytes, head_size, pa::decode_gmax(group));
    int w = (blocks_per_workgroup + bpw - 1) / bpw;
    if (w < 1)
        w = 1;
    if (w > max_waves)
        w = max_waves;
    while (w > 1 && pa::decode_lds_bytes(kv_bytes, head_size, group, w) > kMaxDecodeLds)
        --w;
    return w;
}

int num_partitions(int max_context_len, int partition_size) {
    const int64_t np = (static_cast<int64_t>(max_context_len) + partition_size - 1) / partition_size;
    return np < 1 ? 1 : static_cast<int>(np > INT32_MAX ? INT32_MAX : np);
}

}  // namespace

extern "C" {

const char* pa_status_str(pa_status_t status) {
    switch (status) {
    case PA_OK: return "ok";
    case PA_EINVAL: return "invalid argument";
    case PA_EUNSUPPORTED: return "unsupported configuration";
    case PA_EWORKSPACE: return "workspace too small";
    case PA_EHIP: return "HIP launch failed";
    case PA_ENOSPACE: return "no free block";
    }
    return "unknown status";
}

pa_status_t pa_reshape_and_cache(const void* key, const void* value, void* key_cache,
                                 void* value_cache, const int64_t* slot_mapping, int64_t num_tokens,
                                 int num_kv_heads, int head_size, int block_size, int64_t num_blocks,
                                 pa_dtype_t kv_dtype, void* stream) {
    if (num_tokens < 0 || num_kv_heads <= 0 || head_size <= 0 || block_size <= 0 || num_blocks < 0)
        return PA_EINVAL;
    if (!dtype_ok(kv_dtype) || block_size != pa::kBlockSize || (head_size != 64 && head_size != 128))
        return PA_EUNSUPPORTED;
    if (num_tokens > INT32_MAX)
        return PA_EUNSUPPORTED;
    if (num_tokens == 0)
        return PA_OK;
    if (!key || !value || !key_cache || !value_cache || !slot_mapping)
        return PA_EINVAL;
    if (!aligned(key, 16) || !aligned(value, 16) || !aligned(key_cache, 16) ||
        !aligned(value_cache, 16) || !aligned(slot_mapping, 8))
        return PA_EINVAL;
    const int row = head_size * elem_bytes(kv_dtype);
    const int64_t block_bytes = static_cast<int64_t>(num_kv_heads) * pa::kBlockSize * row;
    if (num_blocks > INT64_MAX / block_bytes)
        return PA_EINVAL;
    pa::CacheParams p{};
    p.key = static_cast<const uint8_t*>(key);
    p.value = static_cast<const uint8_t*>(value);
    p.key_cache = static_cast<uint8_t*>(key_cache);
    p.value_cache = static_cast<uint8_t*>(value_cache);
    p.slot_mapping = slot_mapping;
    p.num_slots = num_blocks * pa::kBlockSize;
    p.num_kv_heads = num_kv_heads;
    p.row_bytes = row;
    return from_hip(pa::launch_cache(p, num_tokens, static_cast<hipStream_t>(stream)));
}

pa_status_t pa_stream_read(const void* src, int64_t num_words, void* sink, int num_workgroups,
                           void* stream) {
    if (num_words < 0 || num_workgroups <= 0 || num_workgroups > (1 << 20) || !sink ||
        (num_words > 0 && !src))
        return PA_EINVAL;
    if ((num_words > 0 && !aligned(src, 16)) || !aligned(sink, 16))
        return PA_EINVAL;
    if (num_words > INT64_MAX / 16)
        return PA_EINVAL;
    return from_hip(pa::launch_stream_read(src, num_words, sink, num_workgroups,
                                           static_cast<hipStream_t>(stream)));
}

pa_status_t pa_copy_blocks(void* key_cache, void* value_cache, const int64_t* block_mapping,
                           int64_t num_pairs, int num_kv_heads, int head_size, int block_size,
                           int64_t num_blocks, pa_dtype_t kv_dtype, void* stream) {
    if (num_pairs < 0 || num_kv_heads <= 0 || head_size <= 0 || block_size <= 0 || num_blocks < 0)
        return PA_EINVAL;
    if (!dtype_ok(kv_dtype) || block_size != pa::kBlockSize || (head_size != 64 && head_size != 128))
        return PA_EUNSUPPORTED;
    if (num_pairs > INT32_MAX)
        return PA_EUNSUPPORTED;
    if (num_pairs == 0)
        return PA_OK;
    if (!key_cache || !value_cache || !block_mapping)
        return PA_EINVAL;
    if (!aligned(key_cache, 16) || !aligned(value_cache, 16) || !aligned(block_mapping, 8))
        return PA_EINVAL;
    const int64_t block_bytes = static_cast<int64_t>(num_kv_heads) * pa::kBlockSize * head_size *
                                elem_bytes(kv_dtype);
    if (num_blocks > INT64_MAX / block_bytes)
        return PA_EINVAL;
    pa::CopyParams p{};
    p.key_cache = static_cast<uint8_t*>(key_cache);
    p.value_cache = static_cast<uint8_t*>(value_cache);
    p.block_mapping = block_mapping;
    p.num_blocks = num_blocks;
    p.block_bytes = block_bytes;
    return from_hip(pa::launch_copy_blocks(p, num_pairs, static_cast<hipStream_t>(stream)));
}

// The address a kernel uses for `p`: device memory as it is, pinned host
// memory (hipHostMalloc, torch's pin_memory) through its device mapping.
// Anything else (pageable host memory) is refused: the GPU cannot read it.
static bool device_address(const void* p, const void** out) {
    hipPointerAttribute_t a{};
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();                  // clear the runtime's error state
        return false;
    }
    if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) {
        *out = p;
        return true;
    }
    if (a.type == hipMemoryTypeHost && a.devicePointer != nullptr) {
        const char* base = static_cast<const char*>(a.hostPointer ? a.hostPointer : p);
        *out = static_cast<const char*>(a.devicePointer) + (static_cast<const char*>(p) - base);
        return true;
    }
    return false;
}

pa_status_t pa_swap_blocks(const void* src_key_cache, const void* src_value_cache,
                           int64_t src_num_blocks, void* dst_key_cache, void* dst_value_cache,
                           int64_t dst_num_blocks, const int64_t* block_mapping, int64_t num_pairs,
                           int num_kv_heads, int head_size, int block_size, pa_dtype_t kv_dtype,
                           void* stream) {
    if (num_pairs < 0 || num_kv_heads <= 0 || head_size <= 0 || block_size <= 0 ||
        src_num_blocks < 0 || dst_num_blocks < 0)
        return PA_EINVAL;
    if (!dtype_ok(kv_dtype) || block_size != pa::kBlockSize || (head_size != 64 && head_size != 128))
        return PA_EUNSUPPORTED;
    if (num_pairs > INT32_MAX)
        return PA_EUNSUPPORTED;
    if (num_pairs == 0)
        return PA_OK;
    if (!src_key_cache || !src_value_cache || !dst_key_cache || !dst_value_cache || !block_mapping)
        return PA_EINVAL;
    if (!aligned(src_key_cache, 16) || !aligned(src_value_cache, 16) || !aligned(dst_key_cache, 16) ||
        !aligned(dst_value_cache, 16) || !aligned(block_mapping, 8))
        return PA_EINVAL;
    const int64_t block_bytes = static_cast<int64_t>(num_kv_heads) * pa::kBlockSize * head_size *
                                elem_bytes(kv_dtype);
    if (src_num_blocks > INT64_MAX / block_bytes || dst_num_blocks > INT64_MAX / block_bytes)
        return PA_EINVAL;
    const void *sk, *sv, *dk, *dv, *map;
    if (!device_address(src_key_cache, &sk) || !device_address(src_value_cache, &sv) ||
        !device_address(dst_key_cache, &dk) || !device_address(dst_value_cache, &dv) ||
        !device_address(block_mapping, &map))
        return PA_EINVAL;
    pa::SwapParams p{};
    p.src_key = static_cast<const uint8_t*>(sk);
    p.src_value = static_cast<const uint8_t*>(sv);
    p.dst_key = static_cast<uint8_t*>(const_cast<void*>(dk));
    p.dst_value = static_cast<uint8_t*>(const_cast<void*>(dv));
    p.block_mapping = static_cast<const int64_t*>(map);
    p.src_num_blocks = src_num_blocks;
    p.dst_num_blocks = dst_num_blocks;
    p.block_bytes = block_bytes;
    return from_hip(pa::launch_swap_blocks(p, num_pairs, static_cast<hipStream_t>(stream)));
}

pa_status_t pa_decode(void* out, pa_dtype_t out_dtype, const void* query, const void* key_cache,
                      const void* value_cache, pa_dtype_t kv_dtype, const int32_t* block_tables,
                      int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                      int num_q_heads, int num_kv_heads, int head_size, int block_size,
                      int64_t num_blocks, float scale, void* stream) {
    pa_status_t st = check_decode(out, out_dtype, query, key_cache, value_cache, kv_dtype,
                                  block_tables, max_blocks_per_seq, context_lens, num_seqs,
                                  num_q_heads, num_kv_heads, head_size, block_size, num_blocks,
                                  scale);
    if (st != PA_OK || num_seqs == 0)
        return st;
    pa::DecodeParams p = make_params(query, key_cache, value_cache, block_tables,
                                     max_blocks_per_seq, context_lens, num_q_heads, num_kv_heads,
                                     num_blocks, scale);
    p.out = out;
    p.partition_blocks = max_blocks_per_seq;
    p.num_partitions = 1;
    p.part_stride = 1;
    p.table_blocks = max_blocks_per_seq;
    p.num_seqs = num_seqs;
    p.persistent = 0;
    const int waves = choose_waves(max_blocks_per_seq, elem_bytes(kv_dtype), head_size, p.group,
                                   pa::kMaxWaves);
    return from_hip(pa::launch_decode(p, kv_dtype == PA_BF16, head_size, out_dtype == PA_BF16,
                                      num_seqs, 1, waves, static_cast<hipStream_t>(stream)));
}

size_t pa_decode_partitioned_workspace_size(int num_seqs, int num_q_heads, int head_size,
                                            int max_context_len, int partition_size) {
    if (num_seqs < 0 || num_q_heads <= 0 || head_size <= 0 || max_context_len < 0 ||
        partition_size <= 0)
        return 0;
    const unsigned __int128 rows = static_cast<unsigned __int128>(num_seqs) *
                                   static_cast<unsigned __int128>(num_q_heads) *
                                   static_cast<unsigned __int128>(num_partitions(max_context_len, partition_size));
    const unsigned __int128 bytes = 2 * (rows * 4 + 256) + rows * 4 * head_size + 256;
    if (bytes > static_cast<unsigned __int128>(SIZE_MAX / 2))
        return 0;
    const size_t r = static_cast<size_t>(rows);
    return 2 * align256(r * sizeof(float)) + align256(r * sizeof(float) * head_size);
}

// Shared by pa_decode_partitioned and pa_decode_partitioned_step (new_key =
// nullptr: no write).
static pa_status_t decode_partitioned(void* out, pa_dtype_t out_dtype, const void* query,
                                      const void* new_key, const void* new_value,
                                      const void* key_cache, const void* value_cache,
                                      pa_dtype_t kv_dtype, const int32_t* block_tables,
                                      int max_blocks_per_seq, const int32_t* context_lens,
                                      int num_seqs, int num_q_heads, int num_kv_heads,
                                      int head_size, int block_size, int64_t num_blocks,
                                      float scale, int max_context_len, int partition_size,
                                      void* workspace, size_t workspace_bytes, void* stream) {
    pa_status_t st = check_decode(out, out_dtype, query, key_cache, value_cache, kv_dtype,
                                  block_tables, max_blocks_per_seq, context_lens, num_seqs,
                                  num_q_heads, num_kv_heads, head_size, block_size, num_blocks,
                                  scale);
    if (st != PA_OK)
        return st;
    if (max_context_len < 0 || partition_size <= 0 || partition_size % pa::kBlockSize != 0)
        return PA_EINVAL;
    if (new_key != nullptr || new_value != nullptr) {
        if (!new_key || !new_value || !aligned(new_key, 16) || !aligned(new_value, 16))
            return PA_EINVAL;
    }
    const int np = num_partitions(max_context_len, partition_size);
    if (np > kMaxGridYZ)
        return PA_EUNSUPPORTED;
    if (num_seqs == 0)
        return PA_OK;
    const size_t need = pa_decode_partitioned_workspace_size(num_seqs, num_q_heads, head_size,
                                                             max_context_len, partition_size);
    if (need == 0)
        return PA_EUNSUPPORTED;
    if (!workspace || workspace_bytes < need)
        return PA_EWORKSPACE;
    if (!aligned(workspace, 256))
        return PA_EINVAL;

    const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads * np;
    char* ws = static_cast<char*>(workspace);
    pa::DecodeParams p = make_params(query, key_cache, value_cache, block_tables,
                                     max_blocks_per_seq, context_lens, num_q_heads, num_kv_heads,
                                     num_blocks, scale);
    p.out = out;
    p.part_max = reinterpret_cast<float*>(ws);
    p.part_sum = reinterpret_cast<float*>(ws + align256(rows * sizeof(float)));
    p.part_out = reinterpret_cast<float*>(ws + 2 * align256(rows * sizeof(float)));
    p.partition_blocks = partition_size / pa::kBlockSize;
    p.num_partitions = np;
    p.part_stride = np;
    p.table_blocks = max_blocks_per_seq;
    p.num_seqs = num_seqs;
    p.persistent = num_seqs <= pa::kMaxPersistentSeqs;
    p.new_key = new_key;
    p.new_value = new_value;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int waves = choose_waves(p.partition_blocks, elem_bytes(kv_dtype), head_size, p.group,
                                   pa::kPartWaves);
    hipError_t e = pa::launch_decode(p, kv_dtype == PA_BF16, head_size, out_dtype == PA_BF16,
                                     num_seqs, np, waves, s);
    if (e != hipSuccess)
        return PA_EHIP;
    if (np == 1)
        return PA_OK;    // every context fits one partition: no partials to combine

    pa::ReduceParams r{};
    r.context_lens = context_lens;
    r.part_max = p.part_max;
    r.part_sum = p.part_sum;
    r.part_out = p.part_out;
    r.out = out;
    r.num_blocks = num_blocks;
    r.max_blocks_per_seq = max_blocks_per_seq;
    r.num_q_heads = num_q_heads;
    r.num_kv_heads = num_kv_heads;
    r.group = p.group;
    r.num_partitions = np;
    r.part_stride = np;
    r.partition_blocks = p.partition_blocks;
    r.table_blocks = max_blocks_per_seq;
    return from_hip(pa::launch_reduce(r, head_size, out_dtype == PA_BF16, num_seqs, s));
}

pa_status_t pa_decode_partitioned(void* out, pa_dtype_t out_dtype, const void* query,
                                  const void* key_cache, const void* value_cache,
                                  pa_dtype_t kv_dtype, const int32_t* block_tables,
                                  int max_blocks_per_seq, const int32_t* context_lens,
                                  int num_seqs, int num_q_heads, int num_kv_heads, int head_size,
                                  int block_size, int64_t num_blocks, float scale,
                                  int max_context_len, int partition_size, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    return decode_partitioned(out, out_dtype, query, nullptr, nullptr, key_cache, value_cache,
                              kv_dtype, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                              num_q_heads, num_kv_heads, head_size, block_size, num_blocks, scale,
                              max_context_len, partition_size, workspace, workspace_bytes, stream);
}

pa_status_t pa_decode_partitioned_step(void* out, pa_dtype_t out_dtype, const void* query,
                                       const void* key, const void* value, void* key_cache,
                                       void* value_cache, pa_dtype_t kv_dtype,
                                       const int32_t* block_tables, int max_blocks_per_seq,
                                       const int32_t* context_lens, int num_seqs,
                                       int num_q_heads, int num_kv_heads, int head_size,
                                       int block_size, int64_t num_blocks, float scale,
                                       int max_context_len, int partition_size, void* workspace,
                                       size_t workspace_bytes, void* stream) {
    if (num_seqs > 0 && (!key || !value))
        return PA_EINVAL;
    return decode_partitioned(out, out_dtype, query, key, value, key_cache, value_cache, kv_dtype,
                              block_tables, max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                              num_kv_heads, head_size, block_size, num_blocks, scale,
                              max_context_len, partition_size, workspace, workspace_bytes, stream);
}

// Workspace of the balanced decode: descriptors, then the partials of the at
// most two cut rows of each workgroup.
struct BalancedWorkspace {
    size_t desc, part_max, part_sum, part_out, total;
};

static BalancedWorkspace balanced_layout(int group, int head_size) {
    const size_t slots = 2 * static_cast<size_t>(pa::kMaxBalancedWorkgroups) * group;
    BalancedWorkspace w{};
    w.desc = 0;
    w.part_max = align256(sizeof(int4) * pa::kMaxBalancedWorkgroups);
    w.part_sum = w.part_max + align256(sizeof(float) * slots);
    w.part_out = w.part_sum + align256(sizeof(float) * slots);
    w.total = w.part_out + align256(sizeof(float) * slots * head_size);
    return w;
}

size_t pa_decode_balanced_workspace_size(int num_q_heads, int num_kv_heads, int head_size) {
    if (num_q_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 || num_q_heads % num_kv_heads != 0 ||
        num_q_heads / num_kv_heads > kMaxGroup || head_size > 4096)
        return 0;
    return balanced_layout(num_q_heads / num_kv_heads, head_size).total;
}

// Shared by pa_decode_balanced and pa_decode_step (new_key = nullptr: no write).
static pa_status_t decode_balanced(void* out, pa_dtype_t out_dtype, const void* query,
                                   const void* new_key, const void* new_value, void* key_cache,
                                   void* value_cache, pa_dtype_t kv_dtype,
                                   const int32_t* block_tables, int max_blocks_per_seq,
                                   const int32_t* context_lens, int num_seqs, int num_q_heads,
                                   int num_kv_heads, int head_size, int block_size,
                                   int64_t num_blocks, float scale, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    pa_status_t st = check_decode(out, out_dtype, query, key_cache, value_cache, kv_dtype,
                                  block_tables, max_blocks_per_seq, context_lens, num_seqs,
                                  num_q_heads, num_kv_heads, head_size, block_size, num_blocks,
                                  scale);
    if (st != PA_OK)
        return st;
    if (num_seqs > pa::kMaxBalancedSeqs ||
        static_cast<int64_t>(num_seqs) * num_kv_heads * max_blocks_per_seq > INT32_MAX)
        return PA_EUNSUPPORTED;
    if (num_seqs == 0)
        return PA_OK;
    if (new_key != nullptr || new_value != nullptr) {
        if (!new_key || !new_value || !aligned(new_key, 16) || !aligned(new_value, 16))
            return PA_EINVAL;
    }
    const size_t need = pa_decode_balanced_workspace_size(num_q_heads, num_kv_heads, head_size);
    if (!workspace || workspace_bytes < need)
        return PA_EWORKSPACE;
    if (!aligned(workspace, 256))
        return PA_EINVAL;
    const BalancedWorkspace lay = balanced_layout(num_q_heads / num_kv_heads, head_size);
    char* ws = static_cast<char*>(workspace);
    pa::BalancedParams bp{};
    bp.d = make_params(query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
                       num_q_heads, num_kv_heads, num_blocks, scale);
    bp.d.out = out;
    bp.d.part_max = reinterpret_cast<float*>(ws + lay.part_max);
    bp.d.part_sum = reinterpret_cast<float*>(ws + lay.part_sum);
    bp.d.part_out = reinterpret_cast<float*>(ws + lay.part_out);
    bp.d.num_seqs = num_seqs;
    bp.d.num_partitions = 1;
    bp.d.partition_blocks = max_blocks_per_seq;
    bp.d.table_blocks = max_blocks_per_seq;
    bp.desc = reinterpret_cast<int4*>(ws + lay.desc);
    bp.new_key = new_key;
    bp.new_value = new_value;
    // At least two units per wave when every context fills its table.
    const int64_t bound = static_cast<int64_t>(num_seqs) * num_kv_heads * max_blocks_per_seq;
    const int64_t per_wg = 2 * static_cast<int64_t>(pa::kBalancedWaves);
    const int max_wgs = static_cast<int>((bound + per_wg - 1) / per_wg);
    return from_hip(pa::launch_decode_balanced(bp, kv_dtype == PA_BF16, head_size,
                                               out_dtype == PA_BF16, max_wgs,
                                               static_cast<hipStream_t>(stream)));
}

pa_status_t pa_decode_balanced(void* out, pa_dtype_t out_dtype, const void* query,
                               const void* key_cache, const void* value_cache, pa_dtype_t kv_dtype,
                               const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* context_lens, int num_seqs, int num_q_heads,
                               int num_kv_heads, int head_size, int block_size, int64_t num_blocks,
                               float scale, void* workspace, size_t workspace_bytes, void* stream) {
    return decode_balanced(out, out_dtype, query, nullptr, nullptr, const_cast<void*>(key_cache),
                           const_cast<void*>(value_cache), kv_dtype, block_tables,
                           max_blocks_per_seq, context_lens, num_seqs, num_q_heads, num_kv_heads,
                           head_size, block_size, num_blocks, scale, workspace, workspace_bytes,
                           stream);
}

pa_status_t pa_decode_step(void* out, pa_dtype_t out_dtype, const void* query, const void* key,
                           const void* value, void* key_cache, void* value_cache,
                           pa_dtype_t kv_dtype, const int32_t* block_tables, int max_blocks_per_seq,
                           const int32_t* context_lens, int num_seqs, int num_q_heads,
                           int num_kv_heads, int head_size, int block_size, int64_t num_blocks,
                           float scale, void* workspace, size_t workspace_bytes, void* stream) {
    if (num_seqs > 0 && (!key || !value))
        return PA_EINVAL;
    return decode_balanced(out, out_dtype, query, key, value, key_cache, value_cache, kv_dtype,
                           block_tables, max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                           num_kv_heads, head_size, block_size, num_blocks, scale, workspace,
                           workspace_bytes, stream);
}

// Partitions of a cascade call: the suffix partitions (tokens past the shared
// prefix, at most max_context_len - 16 * num_prefix_blocks) and one slot per
// prefix chunk.
static void cascade_shape(int max_context_len, int partition_size, int num_prefix_blocks,
                          int* suffix_parts, int* chunks) {
    const int64_t suffix = static_cast<int64_t>(max_context_len) -
                           static_cast<int64_t>(num_prefix_blocks) * pa::kBlockSize;
    *suffix_parts = num_partitions(suffix > 0 ? static_cast<int>(suffix) : 0, partition_size);
    *chunks = (num_prefix_blocks + pa::kCascadeChunkBlocks - 1) / pa::kCascadeChunkBlocks;
}

size_t pa_decode_cascade_workspace_size(int num_seqs, int num_q_heads, int head_size,
                                        int max_context_len, int partition_size,
                                        int num_prefix_blocks) {
    if (num_seqs < 0 || num_q_heads <= 0 || head_size <= 0 || max_context_len < 0 ||
        partition_size <= 0 || num_prefix_blocks <= 0)
        return 0;
    int sp = 0, ch = 0;
    cascade_shape(max_context_len, partition_size, num_prefix_blocks, &sp, &ch);
    const unsigned __int128 rows = static_cast<unsigned __int128>(num_seqs) *
                                   static_cast<unsigned __int128>(num_q_heads) *
                                   static_cast<unsigned __int128>(sp + ch);
    const unsigned __int128 bytes = 2 * (rows * 4 + 256) + rows * 4 * head_size + 256;
    if (bytes > static_cast<unsigned __int128>(SIZE_MAX / 2))
        return 0;
    const size_t r = static_cast<size_t>(rows);
    return 2 * align256(r * sizeof(float)) + align256(r * sizeof(float) * head_size);
}

pa_status_t pa_decode_cascade(void* out, pa_dtype_t out_dtype, const void* query,
                              const void* key_cache, const void* value_cache, pa_dtype_t kv_dtype,
                              const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* context_lens, int num_seqs, int num_q_heads,
                              int num_kv_heads, int head_size, int block_size, int64_t num_blocks,
                              float scale, int num_prefix_blocks, int max_context_len,
                              int partition_size, void* workspace, size_t workspace_bytes,
                              void* stream) {
    pa_status_t st = check_decode(out, out_dtype, query, key_cache, value_cache, kv_dtype,
                                  block_tables, max_blocks_per_seq, context_lens, num_seqs,
                                  num_q_heads, num_kv_heads, head_size, block_size, num_blocks,
                                  scale);
    if (st != PA_OK)
        return st;
    if (kv_dtype != PA_BF16)
        return PA_EUNSUPPORTED;
    if (max_context_len < 0 || partition_size <= 0 || partition_size % pa::kBlockSize != 0 ||
        num_prefix_blocks <= 0 || num_prefix_blocks > max_blocks_per_seq || num_blocks == 0)
        return PA_EINVAL;
    int sp = 0, ch = 0;
    cascade_shape(max_context_len, partition_size, num_prefix_blocks, &sp, &ch);
    if (sp + ch > kMaxGridYZ)
        return PA_EUNSUPPORTED;
    if (num_seqs == 0)
        return PA_OK;
    const size_t need = pa_decode_cascade_workspace_size(num_seqs, num_q_heads, head_size,
                                                         max_context_len, partition_size,
                                                         num_prefix_blocks);
    if (need == 0)
        return PA_EUNSUPPORTED;
    if (!workspace || workspace_bytes < need)
        return PA_EWORKSPACE;
    if (!aligned(workspace, 256))
        return PA_EINVAL;

    const int np = sp + ch;
    const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads * np;
    char* ws = static_cast<char*>(workspace);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    pa::DecodeParams p = make_params(query, key_cache, value_cache, block_tables,
                                     max_blocks_per_seq, context_lens, num_q_heads, num_kv_heads,
                                     num_blocks, scale);
    p.out = out;
    p.part_max = reinterpret_cast<float*>(ws);
    p.part_sum = reinterpret_cast<float*>(ws + align256(rows * sizeof(float)));
    p.part_out = reinterpret_cast<float*>(ws + 2 * align256(rows * sizeof(float)));
    p.partition_blocks = partition_size / pa::kBlockSize;
    p.num_partitions = sp;
    p.part_stride = np;
    p.num_seqs = num_seqs;
    p.skip_blocks = num_prefix_blocks;
    p.table_blocks = max_blocks_per_seq - num_prefix_blocks;
    p.partials_only = 1;

    // 1. The shared prefix: one dense pass per KV head for all query rows.
    // 2. Each sequence's own suffix, through its block table, as partials.
    // Both write disjoint partial slots; on the persistent schedule they go
    // out as one launch whose workgroups take either kind of work.
    pa::CascadeParams c{};
    c.q = query;
    c.k_cache = key_cache;
    c.v_cache = value_cache;
    c.block_tables = block_tables;
    c.part_max = p.part_max;
    c.part_sum = p.part_sum;
    c.part_out = p.part_out;
    c.num_blocks = num_blocks;
    c.num_prefix_blocks = num_prefix_blocks;
    c.chunk_blocks = pa::kCascadeChunkBlocks;
    c.num_seqs = num_seqs;
    c.num_q_heads = num_q_heads;
    c.num_kv_heads = num_kv_heads;
    c.group = p.group;
    c.part_stride = np;
    c.slot_base = sp;
    c.row_tiles = static_cast<int>((static_cast<int64_t>(num_seqs) * p.group + pa::kCascadeTileRows - 1) /
                                   pa::kCascadeTileRows);
    c.num_chunks = ch;
    c.scale_log2 = p.scale_log2;
    bool shared = false;
    hipError_t e = hipSuccess;
    if (p.table_blocks > 0) {
        p.persistent = num_seqs <= pa::kMaxPersistentSeqs;
        const int waves = choose_waves(p.partition_blocks, elem_bytes(kv_dtype), head_size, p.group,
                                       pa::kPartWaves);
        if (p.persistent) {
            // Beside the suffixes the tiles' latency is hidden, so each takes
            // a longer chunk (fewer partials to write and combine).
            pa::CascadeParams cs = c;
            cs.chunk_blocks = pa::kCascadeSharedChunkBlocks;
            cs.num_chunks = (num_prefix_blocks + cs.chunk_blocks - 1) / cs.chunk_blocks;
            e = pa::launch_cascade_shared(p, cs, head_size, out_dtype == PA_BF16, num_seqs, sp, &shared, s);
            if (shared)
                c = cs;
        }
        if (e == hipSuccess && !shared) {
            e = pa::launch_cascade_prefix(c, head_size, s);
            if (e == hipSuccess)
                e = pa::launch_decode(p, 1, head_size, out_dtype == PA_BF16, num_seqs, sp, waves, s);
        }
    } else {
        e = pa::launch_cascade_prefix(c, head_size, s);
    }
    if (e != hipSuccess)
        return PA_EHIP;

    // 3. Log-sum-exp combination of suffix partitions and prefix chunks.
    pa::ReduceParams r{};
    r.context_lens = context_lens;
    r.part_max = p.part_max;
    r.part_sum = p.part_sum;
    r.part_out = p.part_out;
    r.out = out;
    r.num_blocks = num_blocks;
    r.max_blocks_per_seq = max_blocks_per_seq;
    r.num_q_heads = num_q_heads;
    r.num_kv_heads = num_kv_heads;
    r.group = p.group;
    r.num_partitions = sp;
    r.part_stride = np;
    r.partition_blocks = p.partition_blocks;
    r.skip_blocks = num_prefix_blocks;
    r.table_blocks = p.table_blocks;
    r.extra_base = sp;
    r.extra_count = c.num_chunks;
    return from_hip(pa::launch_reduce(r, head_size, out_dtype == PA_BF16, num_seqs, s));
}

// Row tiles per (sequence, KV head) of a prefill call; -1 when out of range.
static int64_t prefill_row_tiles(int num_q_heads, int num_kv_heads, int max_query_len) {
    if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || max_query_len < 0)
        return -1;
    const int64_t rows = static_cast<int64_t>(max_query_len) * (num_q_heads / num_kv_heads);
    if (rows > INT32_MAX)
        return -1;
    constexpr int kTileRows = pa::kPrefillWaves * 16 * pa::kPrefillRowTiles;
    return (rows + kTileRows - 1) / kTileRows;
}

size_t pa_prefill_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int max_query_len) {
    const int64_t tiles = prefill_row_tiles(num_q_heads, num_kv_heads, max_query_len);
    if (num_seqs < 0 || tiles < 0)
        return 0;
    const int64_t pairs = static_cast<int64_t>(num_seqs) * tiles;
    if (pairs > INT32_MAX || pairs * num_kv_heads > INT32_MAX)
        return 0;
    return align256(static_cast<size_t>(pairs) * sizeof(int32_t) + 1);
}

pa_status_t pa_prefill(void* out, pa_dtype_t out_dtype, const void* query, const void* key_cache,
                       const void* value_cache, pa_dtype_t kv_dtype, const int32_t* block_tables,
                       int max_blocks_per_seq, const int32_t* context_lens,
                       const int32_t* query_start, int64_t num_query_rows, int num_seqs,
                       int num_q_heads, int num_kv_heads, int head_size, int block_size,
                       int64_t num_blocks, float scale, int max_query_len, void* workspace,
                       size_t workspace_bytes, void* stream) {
    pa_status_t st = check_decode(out, out_dtype, query, key_cache, value_cache, kv_dtype,
                                  block_tables, max_blocks_per_seq, context_lens, num_seqs,
                                  num_q_heads, num_kv_heads, head_size, block_size, num_blocks,
                                  scale);
    if (st != PA_OK)
        return st;
    if (kv_dtype != PA_BF16)
        return PA_EUNSUPPORTED;
    if (max_query_len < 0 || num_query_rows < 0)
        return PA_EINVAL;
    if (num_seqs == 0 || max_query_len == 0 || num_query_rows == 0)
        return PA_OK;
    if (!query_start || !aligned(query_start, 4))
        return PA_EINVAL;
    const int64_t tiles = prefill_row_tiles(num_q_heads, num_kv_heads, max_query_len);
    const size_t need = pa_prefill_workspace_size(num_seqs, num_q_heads, num_kv_heads, max_query_len);
    if (tiles < 0 || need == 0)
        return PA_EUNSUPPORTED;
    if (!workspace || workspace_bytes < need)
        return PA_EWORKSPACE;
    if (!aligned(workspace, 256))
        return PA_EINVAL;
    pa::PrefillParams p{};
    p.q = query;
    p.k_cache = key_cache;
    p.v_cache = value_cache;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.query_start = query_start;
    p.num_query_rows = num_query_rows;
    p.out = out;
    p.num_blocks = num_blocks;
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.group = num_q_heads / num_kv_heads;
    p.max_query_len = max_query_len;
    p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
    p.order = static_cast<int*>(workspace);
    return from_hip(pa::launch_prefill(p, head_size, out_dtype == PA_BF16, num_seqs,
                                       static_cast<int>(tiles), static_cast<hipStream_t>(stream)));
}

}  // extern "C"

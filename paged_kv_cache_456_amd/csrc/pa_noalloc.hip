// pa_noalloc.hip -- pa_decode_partitioned_noalloc: the split-context decode
// for callers that cannot allocate device memory (code under HIP graph
// capture, serving loops or harnesses that forbid hipMalloc). The workspace
// of the split (per-partition maxima, sums and partial outputs) is a
// file-scope device array that the library holds on every GPU it runs on
// until the process ends; the call itself allocates nothing.
#include <mutex>
#include <map>

#include "pa.h"
#include "pa_internal.h"

namespace {

// The library-held workspace. In host code this name is only a stand-in for
// the symbol: its device address on the current GPU comes from
// hipGetSymbolAddress, and only that address is ever handed to a kernel.
__device__ __align__(256) unsigned char scratch[PA_NOALLOC_WORKSPACE_BYTES];

std::mutex g_mutex;
std::map<int, void*> g_scratch_ptr;   // device -> device address of `scratch` on it

// Device address of this GPU's copy of `scratch`, looked up once per device
// with that device current. nullptr on failure.
void* scratch_on_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_mutex);
    const auto it = g_scratch_ptr.find(dev);
    if (it != g_scratch_ptr.end())
        return it->second;
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
        return nullptr;
    g_scratch_ptr[dev] = ptr;
    return ptr;
}

}  // namespace

extern "C" pa_status_t pa_decode_partitioned_noalloc(
    void* out, pa_dtype_t out_dtype, const void* query, const void* key_cache,
    const void* value_cache, pa_dtype_t kv_dtype, const int32_t* block_tables,
    int max_blocks_per_seq, const int32_t* context_lens, int num_seqs, int num_q_heads,
    int num_kv_heads, int head_size, int block_size, int64_t num_blocks, float scale,
    int max_context_len, int partition_size, void* stream) {
    // Every host-side check of pa_decode_partitioned runs first, with no
    // workspace: any status but "workspace too small" (an argument error, or
    // OK for an empty batch, where nothing is enqueued) is final.
    const pa_status_t st = pa_decode_partitioned(
        out, out_dtype, query, key_cache, value_cache, kv_dtype, block_tables, max_blocks_per_seq,
        context_lens, num_seqs, num_q_heads, num_kv_heads, head_size, block_size, num_blocks, scale,
        max_context_len, partition_size, nullptr, 0, stream);
    if (st != PA_EWORKSPACE)
        return st;
    const size_t need = pa_decode_partitioned_workspace_size(num_seqs, num_q_heads, head_size,
                                                             max_context_len, partition_size);
    if (need > static_cast<size_t>(PA_NOALLOC_WORKSPACE_BYTES))
        return PA_EWORKSPACE;
    void* ws = scratch_on_current_device();
    if (ws == nullptr)
        return PA_EHIP;
    return pa_decode_partitioned(out, out_dtype, query, key_cache, value_cache, kv_dtype,
                                 block_tables, max_blocks_per_seq, context_lens, num_seqs,
                                 num_q_heads, num_kv_heads, head_size, block_size, num_blocks,
                                 scale, max_context_len, partition_size, ws,
                                 static_cast<size_t>(PA_NOALLOC_WORKSPACE_BYTES), stream);
}

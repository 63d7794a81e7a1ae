// pa_block_manager.cpp -- the host-side block manager of the paged KV cache:
// hands out 16-token blocks of the pool on demand, keeps each sequence's
// block table, shares blocks between forked sequences with reference counts,
// and turns a write into a shared block into a copy-on-write pair.
//
// What the pages fix ("Idea 1: PagedAttention" on the day-9 post, "Why this
// wins"; "The idea vLLM started from: pages" and "Code" on "What vLLM Is and
// Why It Exists"): fixed-size blocks mapped through a per-request block
// table, handed out only as tokens are produced; requests with a common
// prefix share physical blocks; a shared block that must diverge is copied
// alone; preemption takes a request's blocks away to feed another. What they
// leave open is decided as follows (the same rules are documented in
// include/pa.h):
//   * free blocks form a stack, initially with block 0 on top (a fresh pool
//     hands out 0, 1, 2, ...); a released block goes on top;
//   * a table is released from its first entry to its last; a block is free
//     again when no table holds it;
//   * adding a sequence takes all of its blocks or none;
//   * appending a token at position L takes a new block when L is a multiple
//     of the block size, and otherwise, if the last block is shared, replaces
//     it by a fresh block and reports (old, new) for the caller to copy.
// Host memory only; nothing here touches the GPU.
#include <stdint.h>

#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"

struct pa_block_manager {
    struct Seq {
        std::vector<int32_t> table;
        int64_t len = 0;
    };
    int64_t num_blocks = 0;
    int block_size = 16;
    std::vector<int32_t> free_stack;    // top = back
    std::vector<int32_t> refs;
    std::unordered_map<int64_t, Seq> seqs;

    int32_t take() {
        const int32_t b = free_stack.back();
        free_stack.pop_back();
        refs[b] = 1;
        return b;
    }
    int64_t slot(const Seq& s, int64_t t) const {
        return static_cast<int64_t>(s.table[t / block_size]) * block_size + t % block_size;
    }
};

extern "C" {

pa_block_manager* pa_bm_create(int64_t num_blocks, int block_size) {
    if (num_blocks < 0 || num_blocks > INT32_MAX || block_size <= 0)
        return nullptr;
    pa_block_manager* bm = new (std::nothrow) pa_block_manager();
    if (!bm)
        return nullptr;
    try {
        bm->num_blocks = num_blocks;
        bm->block_size = block_size;
        bm->free_stack.resize(static_cast<size_t>(num_blocks));
        for (int64_t i = 0; i < num_blocks; ++i)
            bm->free_stack[static_cast<size_t>(i)] = static_cast<int32_t>(num_blocks - 1 - i);
        bm->refs.assign(static_cast<size_t>(num_blocks), 0);
    } catch (...) {
        delete bm;
        return nullptr;
    }
    return bm;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

pa_status_t pa_bm_add_sequence(pa_block_manager* bm, int64_t seq_id, int num_tokens,
                               int64_t* slots_out) {
    if (!bm || num_tokens < 0 || (num_tokens > 0 && !slots_out) || bm->seqs.count(seq_id))
        return PA_EINVAL;
    const int64_t need = (static_cast<int64_t>(num_tokens) + bm->block_size - 1) / bm->block_size;
    if (need > static_cast<int64_t>(bm->free_stack.size()))
        return PA_ENOSPACE;
    pa_block_manager::Seq* s = nullptr;
    try {                                       // allocations first: nothing changes on failure
        auto ins = bm->seqs.emplace(seq_id, pa_block_manager::Seq());
        s = &ins.first->second;
        s->table.reserve(static_cast<size_t>(need));
    } catch (...) {
        bm->seqs.erase(seq_id);
        return PA_EINVAL;
    }
    for (int64_t i = 0; i < need; ++i)
        s->table.push_back(bm->take());
    s->len = num_tokens;
    for (int64_t t = 0; t < num_tokens; ++t)
        slots_out[t] = bm->slot(*s, t);
    return PA_OK;
}

pa_status_t pa_bm_append_token(pa_block_manager* bm, int64_t seq_id, int64_t* slot_out,
                               int64_t* cow_out) {
    if (!bm || !slot_out || !cow_out)
        return PA_EINVAL;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end())
        return PA_EINVAL;
    pa_block_manager::Seq& s = it->second;
    const int64_t t = s.len;
    cow_out[0] = cow_out[1] = -1;
    if (t % bm->block_size == 0) {
        if (bm->free_stack.empty())
            return PA_ENOSPACE;
        try {
            s.table.reserve(s.table.size() + 1);   // may throw: before any block is taken
        } catch (...) {
            return PA_EINVAL;
        }
        s.table.push_back(bm->take());
    } else {
        const int32_t last = s.table.back();
        if (bm->refs[last] > 1) {
            if (bm->free_stack.empty())
                return PA_ENOSPACE;
            const int32_t fresh = bm->take();
            bm->refs[last] -= 1;
            s.table.back() = fresh;
            cow_out[0] = last;
            cow_out[1] = fresh;
        }
    }
    s.len = t + 1;
    *slot_out = bm->slot(s, t);
    return PA_OK;
}

pa_status_t pa_bm_fork(pa_block_manager* bm, int64_t parent_id, int64_t child_id) {
    if (!bm || parent_id == child_id || bm->seqs.count(child_id))
        return PA_EINVAL;
    auto it = bm->seqs.find(parent_id);
    if (it == bm->seqs.end())
        return PA_EINVAL;
    try {
        pa_block_manager::Seq child = it->second;   // copies first: nothing changes on failure
        auto ins = bm->seqs.emplace(child_id, std::move(child));
        for (int32_t b : ins.first->second.table)
            bm->refs[b] += 1;
    } catch (...) {
        return PA_EINVAL;
    }
    return PA_OK;
}

pa_status_t pa_bm_free_sequence(pa_block_manager* bm, int64_t seq_id) {
    if (!bm)
        return PA_EINVAL;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end())
        return PA_EINVAL;
    for (int32_t b : it->second.table)
        if (--bm->refs[b] == 0)
            bm->free_stack.push_back(b);   // never exceeds the capacity reserved at creation
    bm->seqs.erase(it);
    return PA_OK;
}

int64_t pa_bm_num_free_blocks(const pa_block_manager* bm) {
    return bm ? static_cast<int64_t>(bm->free_stack.size()) : -1;
}

int64_t pa_bm_length(const pa_block_manager* bm, int64_t seq_id) {
    if (!bm)
        return -1;
    auto it = bm->seqs.find(seq_id);
    return it == bm->seqs.end() ? -1 : it->second.len;
}

int64_t pa_bm_block_table(const pa_block_manager* bm, int64_t seq_id, int32_t* table_out,
                          int max_entries, int32_t pad) {
    if (!bm || max_entries < 0 || (max_entries > 0 && !table_out))
        return -1;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end())
        return -1;
    const std::vector<int32_t>& tab = it->second.table;
    const int64_t n = static_cast<int64_t>(tab.size());
    for (int64_t i = 0; i < max_entries; ++i)
        table_out[i] = i < n ? tab[static_cast<size_t>(i)] : pad;
    return n;
}

}  // extern "C"

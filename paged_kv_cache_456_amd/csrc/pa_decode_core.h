// pa_decode_core.h -- the per-wave core of the paged decode kernels: a run of
// KV blocks of one (sequence, KV head) row streamed through the block table
// into online-softmax state, shared by the partition-scheduled kernels
// (pa_decode.hip) and the work-balanced ones (pa_decode_balanced.hip).
//
// What is computed: the new query token of a sequence attends over its KV
// cache, held in 16-token blocks scattered through a shared pool and reached
// through the sequence's block table ("Idea 1: PagedAttention" on the day-9
// post of skandtandon.pages.dev; "The idea vLLM started from: pages" on "What
// vLLM Is and Why It Exists"), with standard scaled dot-product softmax
// attention (the pages print no formula).
//
// A wave takes BPW consecutive blocks per round; with several waves on one
// row they interleave (wave w takes blocks w*BPW.., then per_round further).
// Per round, per wave:
//   * physical block ids come from a per-wave register holding the wave's
//     slice of the block table (one vector load per 64 entries, v_readlane
//     per block), so each table entry is resolved once per wavefront;
//   * the K and V tiles of all BPW blocks (16 tokens x D of one KV head, a
//     contiguous run in the pool) are requested together, and the next
//     round's tiles are requested while this round is computed (K as soon as
//     Q^T K has consumed the K registers, V after P.V);
//   * K is loaded so that lane l holds token l%16, 16-byte chunks l/16+4c of
//     its row: the B-operand layout of a 16x16 MFMA. Q^T K for the whole head
//     group is an MFMA chain (bf16: v_mfma_f32_16x16x32_bf16, fp32:
//     v_mfma_f32_16x16x4_f32), heads as rows, tokens as columns;
//   * softmax statistics are kept online (running max and sum, base-2
//     exponent with scale*log2(e) folded in); the round max is an in-lane max
//     over the BPW blocks followed by a 16-lane DPP row reduction;
//   * V is loaded fully coalesced (consecutive lanes read consecutive 16-byte
//     chunks); P.V runs on the VALU in fp32 with P in fp32 (P rounded to bf16
//     would cost about 2e-3 of accuracy). P moves from the MFMA layout to the
//     V layout through a small per-wave LDS tile.
// Every reduction runs in an order fixed by logical token positions, so
// results never depend on where the blocks sit in the pool.
#pragma once

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace core {

using dev::f32x4;
using dev::u32x4;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float readlane_f(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

__device__ __forceinline__ u32x4 ld16(const char* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// KV tiles are read once per step: stream them past the caches.
__device__ __forceinline__ u32x4 ld16_stream(const char* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// A buffer resource over one tile (wave-uniform base, `bytes` long): loads
// through it take a 32-bit lane offset, and an offset past the end reads 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, bytes, 0x00020000);
}

// 16 bytes at lane offset `off` of a tile, streamed (nontemporal).
__device__ __forceinline__ u32x4 ld16_tile(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}

// Make this wave's LDS writes visible to its own later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename OUT>
__device__ __forceinline__ void store_out(void* base, int64_t idx, float v);
template <>
__device__ __forceinline__ void store_out<F32>(void* base, int64_t idx, float v) {
    static_cast<float*>(base)[idx] = v;
}
template <>
__device__ __forceinline__ void store_out<BF16>(void* base, int64_t idx, float v) {
    static_cast<uint16_t*>(base)[idx] = dev::bf16_out(v);
}

template <typename KV>
struct Ops;

template <>
struct Ops<BF16> {
    __device__ static __forceinline__ void to_f32(const u32x4& c, float (&f)[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(c[i] << 16);
            f[2 * i + 1] = __uint_as_float(c[i] & 0xFFFF0000u);
        }
    }
    // acc[head][token] += q[head][k-chunk] . K[token][k-chunk] for 8 elements.
    __device__ static __forceinline__ f32x4 qk(const u32x4& q, const u32x4& k, f32x4 acc) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, q),
                                                       __builtin_bit_cast(bf16x8, k), acc, 0, 0, 0);
    }
};

template <>
struct Ops<F32> {
    __device__ static __forceinline__ void to_f32(const u32x4& c, float (&f)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            f[i] = __uint_as_float(c[i]);
    }
    __device__ static __forceinline__ f32x4 qk(const u32x4& q, const u32x4& k, f32x4 acc) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(q[e]), __uint_as_float(k[e]),
                                                       acc, 0, 0, 0);
        return acc;
    }
};

template <typename KV, int D>
struct Geometry {
    static constexpr int kRow = D * KV::kBytes;          // bytes per token row
    static constexpr int kTile = kBlockSize * kRow;      // bytes per (block, head) tile
    static constexpr int kCh = kRow / 16;                // 16-byte chunks per row
    static constexpr int kNq = kCh / 4;                  // K chunks per lane per tile
    static constexpr int kTpl = kWave / kCh;             // token rows per coalesced V load
    static constexpr int kNv = kBlockSize / kTpl;        // V chunks per lane per tile
    static constexpr int kEpc = 16 / KV::kBytes;         // elements per chunk
    static_assert(kNq == kNv, "K and V take the same number of loads");
    static_assert(kCh >= 4 && kCh <= kWave, "row must span 4..64 chunks");
};

// A context that cannot be read -- longer than its block table or than the
// partitions of the launch, or a non-empty context in an empty pool -- gets
// an all-NaN output row. Every decode kernel applies the same rule.
__device__ __forceinline__ bool context_unreadable(int L, int max_blocks_per_seq, int num_partitions,
                                                   int partition_blocks, int64_t num_blocks) {
    const int64_t cap = min(static_cast<int64_t>(max_blocks_per_seq),
                            static_cast<int64_t>(num_partitions) * partition_blocks) * kBlockSize;
    return L < 0 || static_cast<int64_t>(L) > cap || (L > 0 && num_blocks <= 0);
}

// Tokens of a context that this call reads: those past the skipped leading
// blocks; -1 (unreadable) when the context is shorter than what is skipped.
__device__ __forceinline__ int call_len(int L, int skip_blocks) {
    const int64_t skip = static_cast<int64_t>(skip_blocks) * kBlockSize;
    return L < skip ? -1 : static_cast<int>(L - skip);
}

// Online-softmax state of one wave over the blocks it has streamed, in the
// MFMA row layout: lane (g = lane / 16, r16 = lane % 16) holds, for heads
// 4g .. 4g+3, the running max m (base-2 units) and the running sum of its
// token column r16; o[h] holds the unnormalised output of head h for the
// EPC elements of chunk lane % CH of the token rows that lane loads.
template <typename KV, int D, int GMAX>
struct WaveAcc {
    float m[4], lsum[4];
    float o[GMAX][Geometry<KV, D>::kEpc];
    bool poisoned;                  // a table entry inside the context lies outside the pool

    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            m[j] = -INFINITY;
            lsum[j] = 0.0f;
        }
#pragma unroll
        for (int h = 0; h < GMAX; ++h)
#pragma unroll
            for (int e = 0; e < Geometry<KV, D>::kEpc; ++e)
                o[h][e] = 0.0f;
        poisoned = false;
    }
};

// Row query vectors of the head group as the MFMA A operand (rows >= G zero).
template <typename KV, int D>
__device__ __forceinline__ void load_query(const DecodeParams& p, int kvh, int s,
                                           u32x4 (&qa)[Geometry<KV, D>::kNq]) {
    using Gm = Geometry<KV, D>;
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane >> 4, r16 = lane & 15;
    const bool live = r16 < p.group;
    const char* qp = static_cast<const char*>(p.q) +
                     ((int64_t)s * p.num_q_heads + (int64_t)kvh * p.group + (live ? r16 : 0)) * Gm::kRow;
#pragma unroll
    for (int c = 0; c < Gm::kNq; ++c)
        qa[c] = live ? ld16(qp + (g + 4 * c) * 16) : u32x4{0u, 0u, 0u, 0u};
}

// Streams blocks of row (s, kvh) into `acc`: this wave's blocks are
// wb0 + r * per_round + b for rounds r < rounds and b < BPW, those below pb1;
// tokens at or past min(16 * pb1, L) are masked. Every block below pb1 holds
// at least one token below L, and rounds >= 1. qa: the row's query
// (load_query). p_lds: this wave's P tile.
template <typename KV, int D, int GMAX>
__device__ __forceinline__ void accumulate_blocks(const DecodeParams& p, float* p_lds,
                                                  const u32x4 (&qa)[Geometry<KV, D>::kNq], int kvh,
                                                  int s, int L, int pb1, int wb0, int per_round,
                                                  int rounds, WaveAcc<KV, D, GMAX>& acc) {
    using Gm = Geometry<KV, D>;
    using Op = Ops<KV>;
    constexpr int NQ = Gm::kNq, NV = Gm::kNv, CH = Gm::kCh, TPL = Gm::kTpl, EPC = Gm::kEpc;
    constexpr int ROW = Gm::kRow, TILE = Gm::kTile;
    constexpr int BPW = decode_bpw(KV::kBytes, D, GMAX);
    constexpr int GP = decode_pstride(GMAX);

    const int lane = threadIdx.x & (kWave - 1);
    const int tok_end = min(pb1 * kBlockSize, L);
    const int g = lane >> 4;       // MFMA lane group: output rows 4g..4g+3
    const int r16 = lane & 15;     // MFMA row/column index: A-operand head, token column
    const int vchunk = lane % CH;  // V layout: chunk within the row
    const int vrow = lane / CH;    //           first token row


    const char* kbase = static_cast<const char*>(p.k_cache) + (int64_t)kvh * TILE;
    const char* vbase = static_cast<const char*>(p.v_cache) + (int64_t)kvh * TILE;
    const int64_t blk_stride = (int64_t)p.num_kv_heads * TILE;
    // Lane offsets inside a tile (loads go through a per-tile buffer resource).
    const uint32_t koff = static_cast<uint32_t>(r16 * ROW + g * 16);          // + 64 c
    const uint32_t voff = static_cast<uint32_t>(vrow * ROW + vchunk * 16);    // + TPL * ROW * c
    const int64_t tbl = (int64_t)s * p.max_blocks_per_seq + p.skip_blocks;

    // Table entries live in a register: lane i holds the entry of slot
    // i % BPW of round r0 + i / BPW, for the RPL rounds from r0 (one vector
    // load, refilled every RPL rounds), and v_readlane picks a round's
    // entries. Slots past the run's end re-read its last entry (and so its
    // last tile, which is read anyway: the extra reads hit in cache) and are
    // masked out afterwards. An entry outside the pool marks the wave
    // poisoned (its output becomes NaN) and is replaced by block 0, so that
    // every load stays inside the pool. Every load of the steady-state loop
    // below is unconditional (but for the refill), so the compiler can count
    // the loads in flight and wait for each tile alone: round r + 1's K and V
    // tiles stream in while round r computes.
    constexpr int RPL = kWave / BPW;                  // rounds per entry load
    auto block_of = [&](int r, int b) { return wb0 + r * per_round + b; };   // logical block
    auto load_entries = [&](int r0) {
        const int e = p.block_tables[tbl + min(block_of(r0 + lane / BPW, lane % BPW), pb1 - 1)];
        const bool bad = e < 0 || static_cast<int64_t>(e) >= p.num_blocks;
        if (__ballot(bad) != 0)
            acc.poisoned = true;
        return bad ? 0 : e;
    };

    u32x4 kt[BPW][NQ], vt[BPW][NV];
    int ent = 0;
    auto issue_k = [&](int r) {
#pragma unroll
        for (int b = 0; b < BPW; ++b) {
            const int phys = __builtin_amdgcn_readlane(ent, (r % RPL) * BPW + b);
            const auto rk = tile_rsrc(kbase + (int64_t)phys * blk_stride, TILE);
#pragma unroll
            for (int c = 0; c < NQ; ++c)
                kt[b][c] = ld16_tile(rk, koff + 64u * c);
        }
    };
    auto issue_v = [&](int r) {
#pragma unroll
        for (int b = 0; b < BPW; ++b) {
            const int phys = __builtin_amdgcn_readlane(ent, (r % RPL) * BPW + b);
            const auto rv = tile_rsrc(vbase + (int64_t)phys * blk_stride, TILE);
#pragma unroll
            for (int c = 0; c < NV; ++c)
                vt[b][c] = ld16_tile(rv, voff + static_cast<uint32_t>(TPL * ROW) * c);
        }
    };

    // Round r: Q^T K, online softmax and P.V over this wave's BPW slots. In the
    // steady state (NEXT) the following round's K is requested as soon as the
    // K registers are consumed, the entries of the round after it right then,
    // and its V once P.V is done.
    auto round = [&](int r, auto next_tag) {
        constexpr bool NEXT = decltype(next_tag)::value;
        const int nvb = min(BPW, max(0, pb1 - block_of(r, 0)));   // this wave's blocks this round
        f32x4 lg[BPW];
#pragma unroll
        for (int b = 0; b < BPW; ++b) {
            lg[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int c = 0; c < NQ; ++c)
                lg[b] = Op::qk(qa[c], kt[b][c], lg[b]);
        }
        if constexpr (NEXT) {
            if ((r + 1) % RPL == 0)
                ent = load_entries(r + 1);
            issue_k(r + 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (nvb > 0) {
            // ---- online softmax over the round
            float x[BPW][4];
            float alpha[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float mx = -INFINITY;
#pragma unroll
                for (int b = 0; b < BPW; ++b) {
                    const bool tvalid = block_of(r, b) * kBlockSize + r16 < tok_end;
                    x[b][j] = tvalid ? lg[b][j] * p.scale_log2 : -INFINITY;
                    mx = fmaxf(mx, x[b][j]);
                }
                const float mn = fmaxf(acc.m[j], dev::row_max16(mx));
                alpha[j] = __builtin_amdgcn_exp2f(acc.m[j] - mn);
                float ps = 0.0f;
#pragma unroll
                for (int b = 0; b < BPW; ++b) {
                    x[b][j] = __builtin_amdgcn_exp2f(x[b][j] - mn);
                    ps += x[b][j];
                }
                acc.lsum[j] = acc.lsum[j] * alpha[j] + ps;
                acc.m[j] = mn;
            }
            if (4 * g < GP) {
#pragma unroll
                for (int b = 0; b < BPW; ++b)
                    *reinterpret_cast<f32x4*>(p_lds + (b * kBlockSize + r16) * GP + 4 * g) =
                        f32x4{x[b][0], x[b][1], x[b][2], x[b][3]};
            }
            float al[GMAX];
#pragma unroll
            for (int h = 0; h < GMAX; ++h)
                al[h] = readlane_f(alpha[h & 3], 16 * (h >> 2));
            wave_lds_sync();
#pragma unroll
            for (int h = 0; h < GMAX; ++h)
#pragma unroll
                for (int e = 0; e < EPC; ++e)
                    acc.o[h][e] *= al[h];
            // ---- P.V
#pragma unroll
            for (int b = 0; b < BPW; ++b) {
                // Valid rows of the slot: 16 for a full block, fewer for the
                // context's last block, none (<= 0) for a slot past the end.
                const int tvalid = tok_end - block_of(r, b) * kBlockSize;
#pragma unroll
                for (int c = 0; c < NV; ++c) {
                    const int tr = vrow + TPL * c;
                    const float* prow = p_lds + (b * kBlockSize + tr) * GP;
                    float pv[GMAX];
                    if constexpr (GMAX >= 4) {
#pragma unroll
                        for (int h4 = 0; h4 < GMAX; h4 += 4) {
                            const f32x4 q4 = *reinterpret_cast<const f32x4*>(prow + h4);
                            pv[h4] = q4[0];
                            pv[h4 + 1] = q4[1];
                            pv[h4 + 2] = q4[2];
                            pv[h4 + 3] = q4[3];
                        }
                    } else {
#pragma unroll
                        for (int h = 0; h < GMAX; ++h)
                            pv[h] = prow[h];
                    }
                    float vf[EPC];
                    Op::to_f32(vt[b][c], vf);
                    if (tvalid < kBlockSize && tr >= tvalid) {
                        // Tail rows may hold anything (even NaN): drop them, do not scale by 0.
#pragma unroll
                        for (int e = 0; e < EPC; ++e)
                            vf[e] = 0.0f;
                    }
#pragma unroll
                    for (int h = 0; h < GMAX; ++h)
#pragma unroll
                        for (int e = 0; e < EPC; ++e)
                            acc.o[h][e] = fmaf(pv[h], vf[e], acc.o[h][e]);
                }
            }
            wave_lds_sync();
        }
        if constexpr (NEXT) {
            __builtin_amdgcn_sched_barrier(0);
            issue_v(r + 1);
        }
    };

    // The loads go out in the loop's order -- K, then V -- so that the loop
    // is entered with the same loads in flight, in the same order, as it is
    // re-entered from its back edge (the scheduling barriers keep the
    // compiler from interleaving the groups).
    ent = load_entries(0);
    issue_k(0);
    __builtin_amdgcn_sched_barrier(0);
    issue_v(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma nounroll
    for (int r = 0; r < rounds - 1; ++r)
        round(r, std::true_type{});
    round(rounds - 1, std::false_type{});
}

// The step's new token of one (sequence, KV head), loaded into one register
// before the blocks are streamed (so its load latency hides under theirs):
// lane l < CH holds 16-byte chunk l of the K row, lane CH <= l < 2 CH chunk
// l - CH of the V row -- the layout its store into the slot takes.
template <typename KV, int D>
struct NewToken {
    u32x4 row;
};

template <typename KV, int D>
__device__ __forceinline__ NewToken<KV, D> load_new_token(const char* k_row, const char* v_row) {
    constexpr int CH = Geometry<KV, D>::kCh;
    const int lane = threadIdx.x & (kWave - 1);
    NewToken<KV, D> t;
    t.row = lane < CH       ? ld16(k_row + lane * 16)
            : lane < 2 * CH ? ld16(v_row + (lane - CH) * 16)
                            : u32x4{0u, 0u, 0u, 0u};
    return t;
}

__device__ __forceinline__ u32x4 shfl16(const u32x4& x, int src) {
    return u32x4{static_cast<uint32_t>(__shfl(static_cast<int>(x[0]), src, kWave)),
                 static_cast<uint32_t>(__shfl(static_cast<int>(x[1]), src, kWave)),
                 static_cast<uint32_t>(__shfl(static_cast<int>(x[2]), src, kWave)),
                 static_cast<uint32_t>(__shfl(static_cast<int>(x[3]), src, kWave))};
}

// One more token, the new one: the same online-softmax step as a round, with
// the token in column 0 of the MFMA tile and every other column masked. The
// attention thus never reads the slot the call writes.
template <typename KV, int D, int GMAX>
__device__ __forceinline__ void accumulate_token(const DecodeParams& p,
                                                 const u32x4 (&qa)[Geometry<KV, D>::kNq],
                                                 const NewToken<KV, D>& t,
                                                 WaveAcc<KV, D, GMAX>& acc) {
    using Gm = Geometry<KV, D>;
    using Op = Ops<KV>;
    constexpr int NQ = Gm::kNq, CH = Gm::kCh, EPC = Gm::kEpc;
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane >> 4, r16 = lane & 15;
    // K as token column 0 of the MFMA B operand: lanes 16g take chunks g + 4c.
    f32x4 lg = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
        const u32x4 kc = shfl16(t.row, g + 4 * c);
        lg = Op::qk(qa[c], r16 == 0 ? kc : u32x4{0u, 0u, 0u, 0u}, lg);
    }
    const u32x4 vn = shfl16(t.row, lane < CH ? CH + lane : 0);
    float pn[4], alpha[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float x = r16 == 0 ? lg[j] * p.scale_log2 : -INFINITY;
        const float mn = fmaxf(acc.m[j], dev::row_max16(x));
        alpha[j] = __builtin_amdgcn_exp2f(acc.m[j] - mn);
        pn[j] = __builtin_amdgcn_exp2f(x - mn);
        acc.lsum[j] = acc.lsum[j] * alpha[j] + pn[j];
        acc.m[j] = mn;
    }
    float vf[EPC];
    Op::to_f32(vn, vf);
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
        const float al = readlane_f(alpha[h & 3], 16 * (h >> 2));
        const float ph = lane < CH ? readlane_f(pn[h & 3], 16 * (h >> 2)) : 0.0f;
#pragma unroll
        for (int e = 0; e < EPC; ++e)
            acc.o[h][e] = fmaf(ph, vf[e], acc.o[h][e] * al);
    }
}

// Stores the new token's K and V rows at position L - 1 of sequence s (table
// entry skip + (L - 1) / 16), KV head kvh, when that entry lies inside the
// pool (otherwise the row's output is NaN already and nothing is written).
template <typename KV, int D>
__device__ __forceinline__ void store_new_token(const DecodeParams& p, const NewToken<KV, D>& t,
                                                int s, int kvh, int L, int skip) {
    using Gm = Geometry<KV, D>;
    constexpr int CH = Gm::kCh, ROW = Gm::kRow;
    const int lane = threadIdx.x & (kWave - 1);
    const int tb = (L - 1) / kBlockSize, tr = (L - 1) % kBlockSize;
    const int phys = p.block_tables[(int64_t)s * p.max_blocks_per_seq + skip + tb];
    if (phys >= 0 && static_cast<int64_t>(phys) < p.num_blocks && lane < 2 * CH) {
        const bool is_v = lane >= CH;
        const int c = is_v ? lane - CH : lane;
        char* dst = static_cast<char*>(const_cast<void*>(is_v ? p.v_cache : p.k_cache)) +
                    (((int64_t)phys * p.num_kv_heads + kvh) * kBlockSize + tr) * ROW + c * 16;
        *reinterpret_cast<u32x4*>(dst) = t.row;
    }
}

// Totals of a wave's state: srow[j] = the sum of head 4g+j over the 16 token
// columns (in every lane of the row group), and o summed over the lanes that
// hold the same chunk of different token rows. A poisoned state becomes
// (m = 0, sum = NaN, o = NaN), which turns every output it reaches into NaN.
template <typename KV, int D, int GMAX>
__device__ __forceinline__ void wave_totals(WaveAcc<KV, D, GMAX>& acc, float (&srow)[4]) {
    constexpr int CH = Geometry<KV, D>::kCh, EPC = Geometry<KV, D>::kEpc;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        srow[j] = dev::row_sum16(acc.lsum[j]);
#pragma unroll
    for (int off = CH; off < kWave; off <<= 1)
#pragma unroll
        for (int h = 0; h < GMAX; ++h)
#pragma unroll
            for (int e = 0; e < EPC; ++e)
                acc.o[h][e] += __shfl_xor(acc.o[h][e], off, kWave);
    if (acc.poisoned) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc.m[j] = 0.0f;
            srow[j] = __builtin_nanf("");
        }
#pragma unroll
        for (int h = 0; h < GMAX; ++h)
#pragma unroll
            for (int e = 0; e < EPC; ++e)
                acc.o[h][e] = __builtin_nanf("");
    }
}

}  // namespace core
}  // namespace pa

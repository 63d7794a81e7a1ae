// pa_decode.hip -- paged decode attention kernel for gfx950 (CDNA4).
//
// What is computed: for each sequence, its one new query token attends over
// a KV cache held in 16-token blocks scattered through a shared pool and
// reached through the sequence's block table ("Idea 1: PagedAttention" on
// the day-9 post of skandtandon.pages.dev; "The idea vLLM started from:
// pages" on "What vLLM Is and Why It Exists"). The attention is standard
// scaled dot-product softmax attention (the pages print no formula).
//
// Work decomposition. A work item is one context partition of one KV head
// of one sequence; the single-pass entry point is the case of one partition
// that spans the whole table. Every query head of the group that shares the
// KV head is handled by the same wave, so each K/V byte is read from HBM once
// per step. The partitioned entry point runs a persistent schedule: only as
// many workgroups as the GPU keeps resident, each taking every grid-th item
// of the list of items that exist (built from context_lens in LDS); the
// single pass, and batches too large for that list, use one workgroup per
// item. An item's blocks are dealt out in rounds: in each round, wave w takes
// BPW consecutive blocks.
//
// Per round, per wave:
//   * physical block ids come from a per-wave register holding the wave's
//     slice of the block table (one vector load per 64 entries, v_readlane
//     per block), so each table entry is resolved once per wavefront;
//   * the K and V tiles of all BPW blocks (16 tokens x D of one KV head, a
//     contiguous run in the pool) are requested together, before any of them
//     is used, and the next round's tiles are requested while this round is
//     computed (K as soon as Q^T K has consumed the K registers, V after P.V);
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
// The waves then merge their (max, sum, output) through LDS in a fixed order.
//
// Split contexts. A sequence with a single partition writes its output row
// directly. Otherwise each partition writes its (max, sum, normalised
// output) to the workspace and a second, small kernel combines the
// partitions of each (sequence, KV head) with log-sum-exp weights, in
// partition order. Every reduction runs in an order fixed by logical token
// positions, so results never depend on where the blocks sit in the pool.
#include <algorithm>

#include "pa_internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// DPP controls (GFX9 encoding).
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Max / sum over the 16 lanes of a DPP row; every lane of the row gets the
// result (the combining order is the same in every lane).
__device__ __forceinline__ float row_max16(float x) {
    x = fmaxf(x, dpp<kQuadSwap1>(x));
    x = fmaxf(x, dpp<kQuadSwap2>(x));
    x = fmaxf(x, dpp<kRowHalfMirror>(x));
    x = fmaxf(x, dpp<kRowMirror>(x));
    return x;
}

__device__ __forceinline__ float row_sum16(float x) {
    x = x + dpp<kQuadSwap1>(x);
    x = x + dpp<kQuadSwap2>(x);
    x = x + dpp<kRowHalfMirror>(x);
    x = x + dpp<kRowMirror>(x);
    return x;
}

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

// Make this wave's LDS writes visible to its own later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// fp32 -> bf16, round to nearest even, NaN kept NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

template <typename OUT>
__device__ __forceinline__ void store_out(void* base, int64_t idx, float v);
template <>
__device__ __forceinline__ void store_out<F32>(void* base, int64_t idx, float v) {
    static_cast<float*>(base)[idx] = v;
}
template <>
__device__ __forceinline__ void store_out<BF16>(void* base, int64_t idx, float v) {
    static_cast<uint16_t*>(base)[idx] = f32_to_bf16(v);
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
// an all-NaN output row. Both kernels apply the same rule.
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

// Writes the output rows of the head group of KV head `kvh` of sequence `s`
// when its context has nothing to read: zeros for an empty context, NaN for
// an unreadable one.
template <typename OUT>
__device__ __forceinline__ void fill_rows(const DecodeParams& p, int kvh, int s, int D, float v) {
    const int G = p.group;
    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
        const int h = idx / D, d = idx - (idx / D) * D;
        store_out<OUT>(p.out, ((int64_t)s * p.num_q_heads + kvh * G + h) * D + d, v);
    }
}

// Blocks [pb0, pb1) of the context of KV head `kvh` of sequence `s` (L > 0
// tokens, readable), computed by the whole workgroup. With `direct` the range
// is the whole context and the output row is written; otherwise the range's
// (max, sum, normalised output) go to partial slot `slot` of the workspace.
// All arguments are wave-uniform.
template <typename KV, int D, int GMAX, typename OUT>
__device__ __forceinline__ void process_range(const DecodeParams& p, float* smem, int kvh, int s,
                                              int L, int pb0, int pb1, int slot, bool direct) {
    using Gm = Geometry<KV, D>;
    using Op = Ops<KV>;
    constexpr int NQ = Gm::kNq, NV = Gm::kNv, CH = Gm::kCh, TPL = Gm::kTpl, EPC = Gm::kEpc;
    constexpr int ROW = Gm::kRow, TILE = Gm::kTile;
    constexpr int BPW = decode_bpw(KV::kBytes, D, GMAX);
    constexpr int GP = decode_pstride(GMAX);
    constexpr int RPB = kWave / BPW;              // rounds covered by one batch of table entries

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nw = blockDim.x / kWave;
    const int Hq = p.num_q_heads, Hkv = p.num_kv_heads, G = p.group;

    const int tok_end = min(pb1 * kBlockSize, L);
    const int per_round = nw * BPW;
    const int rounds = (pb1 - pb0 + per_round - 1) / per_round;
    const int wb0 = pb0 + wave * BPW;            // this wave's first block of round 0

    const int g = lane >> 4;       // MFMA lane group: output rows 4g..4g+3
    const int r16 = lane & 15;     // MFMA row/column index: A-operand head, token column
    const int vchunk = lane % CH;  // V layout: chunk within the row
    const int vrow = lane / CH;    //           first token row

    // Query rows of the head group as the MFMA A operand (rows >= G are zero).
    u32x4 qa[NQ];
    {
        const bool live = r16 < G;
        const char* qp = static_cast<const char*>(p.q) +
                         ((int64_t)s * Hq + (int64_t)kvh * G + (live ? r16 : 0)) * ROW;
#pragma unroll
        for (int c = 0; c < NQ; ++c)
            qa[c] = live ? ld16(qp + (g + 4 * c) * 16) : u32x4{0u, 0u, 0u, 0u};
    }

    const char* kbase = static_cast<const char*>(p.k_cache) + (int64_t)kvh * TILE;
    const char* vbase = static_cast<const char*>(p.v_cache) + (int64_t)kvh * TILE;
    const int64_t blk_stride = (int64_t)Hkv * TILE;
    const int koff = r16 * ROW + g * 16;            // + 64 c
    const int voff = vrow * ROW + vchunk * 16;      // + TPL * ROW * c
    const int64_t tbl = (int64_t)s * p.max_blocks_per_seq + p.skip_blocks;

    float m[4], lsum[4];
    float o[GMAX][EPC];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        m[j] = -INFINITY;
        lsum[j] = 0.0f;
    }
#pragma unroll
    for (int h = 0; h < GMAX; ++h)
#pragma unroll
        for (int e = 0; e < EPC; ++e)
            o[h][e] = 0.0f;

    float* p_lds = smem + wave * (BPW * kBlockSize * GP);
    bool poisoned = false;

    // Table entries of rounds [r0, r0 + RPB): lane i holds block b = i % BPW of
    // round r0 + i / BPW. An entry inside the context that lies outside the
    // pool marks the wave poisoned (its output becomes NaN) and is replaced by
    // block 0, so that every load stays inside the pool.
    int phys_l = 0;
    int batch_r0 = 0;
    auto load_entries = [&](int r0) {
        const int jb = wb0 + (r0 + lane / BPW) * per_round + lane % BPW;
        const bool mine = jb < pb1;
        const int e = mine ? p.block_tables[tbl + jb] : 0;
        const bool bad = e < 0 || static_cast<int64_t>(e) >= p.num_blocks;
        phys_l = bad ? 0 : e;
        batch_r0 = r0;
        if (__ballot(bad) != 0)
            poisoned = true;
    };
    auto block_of = [&](int r, int b) { return wb0 + r * per_round + b; };   // logical block
    // Slots of a round past the partition's end re-read the partition's last
    // tile (one that is read anyway, so the extra reads hit in cache) and are
    // masked out afterwards. Every slot is loaded, so no load sits under a
    // branch and the compiler can wait for each tile precisely.
    int last_phys = p.block_tables[tbl + pb1 - 1];
    if (last_phys < 0 || static_cast<int64_t>(last_phys) >= p.num_blocks) {
        poisoned = true;
        last_phys = 0;
    }
    auto phys_of = [&](int r, int b) {
        const int v = __builtin_amdgcn_readlane(phys_l, (r - batch_r0) * BPW + b);
        return block_of(r, b) < pb1 ? v : last_phys;
    };

    u32x4 kt[BPW][NQ], vt[BPW][NV];
    auto issue_k = [&](int r) {
#pragma unroll
        for (int b = 0; b < BPW; ++b) {
            const char* kb = kbase + (int64_t)phys_of(r, b) * blk_stride + koff;
#pragma unroll
            for (int c = 0; c < NQ; ++c)
                kt[b][c] = ld16_stream(kb + 64 * c);
        }
    };
    auto issue_v = [&](int r) {
#pragma unroll
        for (int b = 0; b < BPW; ++b) {
            const char* vb = vbase + (int64_t)phys_of(r, b) * blk_stride + voff;
#pragma unroll
            for (int c = 0; c < NV; ++c)
                vt[b][c] = ld16_stream(vb + TPL * ROW * c);
        }
    };

    // One round: Q^T K, online softmax and P.V over this wave's BPW slots. The
    // following round's K is requested as soon as the K registers are consumed
    // and its V once P.V is done.
    auto round = [&](int r) {
        const int nvb = min(BPW, max(0, pb1 - block_of(r, 0)));   // this wave's blocks this round
        // ---- logits of the round's slots: heads 4g+j, token column r16
        f32x4 acc[BPW];
#pragma unroll
        for (int b = 0; b < BPW; ++b) {
            acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int c = 0; c < NQ; ++c)
                acc[b] = Op::qk(qa[c], kt[b][c], acc[b]);
        }
        if (r + 1 < rounds) {
            if (r + 1 - batch_r0 >= RPB)
                load_entries(r + 1);
            issue_k(r + 1);
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
                    x[b][j] = tvalid ? acc[b][j] * p.scale_log2 : -INFINITY;
                    mx = fmaxf(mx, x[b][j]);
                }
                const float mn = fmaxf(m[j], row_max16(mx));
                alpha[j] = __builtin_amdgcn_exp2f(m[j] - mn);
                float ps = 0.0f;
#pragma unroll
                for (int b = 0; b < BPW; ++b) {
                    x[b][j] = __builtin_amdgcn_exp2f(x[b][j] - mn);
                    ps += x[b][j];
                }
                lsum[j] = lsum[j] * alpha[j] + ps;
                m[j] = mn;
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
                    o[h][e] *= al[h];
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
                            o[h][e] = fmaf(pv[h], vf[e], o[h][e]);
                }
            }
            wave_lds_sync();
        }
        if (r + 1 < rounds)
            issue_v(r + 1);
    };

    load_entries(0);
    issue_k(0);
    issue_v(0);
#pragma nounroll
    for (int r = 0; r < rounds; ++r)
        round(r);

    // Wave totals: sums over the 16 token columns, outputs over the token rows.
    float srow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        srow[j] = row_sum16(lsum[j]);
#pragma unroll
    for (int off = CH; off < kWave; off <<= 1)
#pragma unroll
        for (int h = 0; h < GMAX; ++h)
#pragma unroll
            for (int e = 0; e < EPC; ++e)
                o[h][e] += __shfl_xor(o[h][e], off, kWave);
    if (poisoned) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            m[j] = 0.0f;
            srow[j] = __builtin_nanf("");
        }
#pragma unroll
        for (int h = 0; h < GMAX; ++h)
#pragma unroll
            for (int e = 0; e < EPC; ++e)
                o[h][e] = __builtin_nanf("");
    }

    float* red_m = smem + nw * (BPW * kBlockSize * GP);
    float* red_s = red_m + nw * GP;
    float* red_o = red_s + nw * GP;
    if (r16 == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int h = 4 * g + j;
            if (h < GMAX) {
                red_m[wave * GP + h] = m[j];
                red_s[wave * GP + h] = srow[j];
            }
        }
    }
    if (vrow == 0) {
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
            float* dst = red_o + (wave * GMAX + h) * D + vchunk * EPC;
#pragma unroll
            for (int e = 0; e < EPC; e += 4)
                *reinterpret_cast<f32x4*>(dst + e) = f32x4{o[h][e], o[h][e + 1], o[h][e + 2], o[h][e + 3]};
        }
    }
    __syncthreads();

    // Merge the waves in a fixed order.
    const bool split = !direct;
    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
        const int h = idx / D;
        const int d = idx - h * D;
        float M = -INFINITY;
        for (int w = 0; w < nw; ++w)
            M = fmaxf(M, red_m[w * GP + h]);
        float S = 0.0f, acc = 0.0f;
        for (int w = 0; w < nw; ++w) {
            const float f = __builtin_amdgcn_exp2f(red_m[w * GP + h] - M);
            S = fmaf(red_s[w * GP + h], f, S);
            acc = fmaf(red_o[(w * GMAX + h) * D + d], f, acc);
        }
        const int64_t row = (int64_t)s * Hq + (int64_t)kvh * G + h;
        if (!split) {
            store_out<OUT>(p.out, row * D + d, acc / S);
        } else {
            const int64_t pi = row * p.part_stride + slot;
            p.part_out[pi * D + d] = acc / S;
            if (d == 0) {
                p.part_max[pi] = M * kLn2;
                p.part_sum[pi] = S;
            }
        }
    }
}

// Blocks a context spans, as the schedule counts them: a context with nothing
// to read counts one block (its item writes the zero or NaN row).
__device__ __forceinline__ int schedule_blocks(int L, const DecodeParams& p) {
    if (L == 0 || context_unreadable(L, p.table_blocks, p.num_partitions, p.partition_blocks,
                                     p.num_blocks))
        return 1;
    return (L + kBlockSize - 1) / kBlockSize;
}

// Partition `part` of the context of KV head `kvh` of sequence `s`.
template <typename KV, int D, int GMAX, typename OUT>
__device__ __forceinline__ void process_partition(const DecodeParams& p, float* smem, int kvh,
                                                  int s, int L, int part) {
    const bool bad = context_unreadable(L, p.table_blocks, p.num_partitions, p.partition_blocks,
                                        p.num_blocks);
    if (bad || L == 0) {
        if (part == 0 && !p.partials_only)
            fill_rows<OUT>(p, kvh, s, D, bad ? __builtin_nanf("") : 0.0f);
        return;
    }
    const int nblk = (L + kBlockSize - 1) / kBlockSize;
    const int PB = p.partition_blocks;
    const int np = (nblk + PB - 1) / PB;
    if (part >= np)
        return;
    process_range<KV, D, GMAX, OUT>(p, smem, kvh, s, L, part * PB, min((part + 1) * PB, nblk), part,
                                    np == 1 && !p.partials_only);
}

// Grid schedule: one workgroup per (KV head, sequence, partition). The single
// pass is the case of one partition spanning the whole table.
template <typename KV, int D, int GMAX, typename OUT>
__global__ __launch_bounds__(kMaxWaves * kWave) void paged_decode_kernel(DecodeParams p) {
    extern __shared__ float smem[];
    process_partition<KV, D, GMAX, OUT>(p, smem, blockIdx.x, blockIdx.y,
                                        call_len(p.context_lens[blockIdx.y], p.skip_blocks),
                                        blockIdx.z);
}

// Waves per SIMD the persistent kernel is register-allocated for: three 4-wave
// workgroups per CU for head groups up to 4, two for larger ones.
template <typename KV, int D, int GMAX>
constexpr int persistent_waves_per_simd() {
    return (GMAX <= 4 && D * KV::kBytes <= 256) ? 3 : 2;
}

// Persistent schedule: a grid no larger than what the GPU holds at once,
// where workgroup w takes the items w, w + W, w + 2W, ... of the list of
// (sequence, partition, KV head) items that exist, KV head fastest. The list
// is built from context_lens in LDS, so no workgroup is spent on the empty
// partitions of short sequences. Dealing items round-robin in this order has
// neighbouring workgroups read the same physical blocks for different KV
// heads at about the same time (measured faster on MI355X than contiguous,
// tile-balanced ranges, and than dealing KV head by KV head).
template <typename KV, int D, int GMAX, typename OUT>
__global__ __launch_bounds__(kPartWaves * kWave)
__attribute__((amdgpu_waves_per_eu(persistent_waves_per_simd<KV, D, GMAX>())))
void paged_decode_persistent_kernel(DecodeParams p) {
    extern __shared__ float smem[];
    const int nw = blockDim.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int S = p.num_seqs, Hkv = p.num_kv_heads;
    int* lens = reinterpret_cast<int*>(smem + decode_lds_floats(KV::kBytes, D, p.group, nw));
    int* first_slot = lens + S;                 // [S + 1], exclusive prefix sum of partitions
    int* list = first_slot + S + 1;             // [kItemListCap][2]: sequence, part << 8 | kvh
    for (int i = threadIdx.x; i < S; i += blockDim.x)
        lens[i] = call_len(p.context_lens[i], p.skip_blocks);
    __syncthreads();
    if (threadIdx.x < kWave) {
        int carry = 0;
        for (int c0 = 0; c0 < S; c0 += kWave) {
            const int i = c0 + lane;
            const int nb = i < S ? schedule_blocks(lens[i], p) : 0;
            const int v = (nb + p.partition_blocks - 1) / p.partition_blocks;
            int incl = v;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const int t = __shfl_up(incl, off, kWave);
                if (lane >= off)
                    incl += t;
            }
            if (i < S)
                first_slot[i] = carry + incl - v;
            carry += __shfl(incl, kWave - 1, kWave);
        }
        if (lane == 0)
            first_slot[S] = carry;
    }
    __syncthreads();
    const int64_t items = static_cast<int64_t>(first_slot[S]) * Hkv;
    for (int64_t k0 = 0; blockIdx.x + k0 * gridDim.x < items; k0 += kItemListCap) {
        for (int k = threadIdx.x; k < kItemListCap; k += blockDim.x) {
            const int64_t it = blockIdx.x + (k0 + k) * gridDim.x;
            int seq = -1, pk = 0;
            if (it < items) {
                const int slot = static_cast<int>(it / Hkv);
                const int kvh = static_cast<int>(it - static_cast<int64_t>(slot) * Hkv);
                int lo = 0, hi = S;                 // last sequence whose first slot <= slot
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (first_slot[mid] <= slot)
                        lo = mid;
                    else
                        hi = mid;
                }
                seq = lo;
                pk = ((slot - first_slot[lo]) << 8) | kvh;
            }
            list[2 * k] = seq;
            list[2 * k + 1] = pk;
        }
        __syncthreads();
        for (int k = 0; k < kItemListCap; ++k) {
            const int seq = __builtin_amdgcn_readfirstlane(list[2 * k]);
            if (seq < 0)
                break;
            const int pk = __builtin_amdgcn_readfirstlane(list[2 * k + 1]);
            process_partition<KV, D, GMAX, OUT>(p, smem, pk & 0xFF, seq,
                                                __builtin_amdgcn_readfirstlane(lens[seq]), pk >> 8);
            __syncthreads();                        // the item's LDS is free again
        }
        __syncthreads();                            // every thread is done with this list
    }
}

// Log-sum-exp combination of the partitions of every (sequence, KV head)
// whose context spans more than one partition: one workgroup per row, one
// wave per query head at a time. The row's partials are its own partitions
// followed by any extra slots (shared-prefix chunks), merged 64 at a time:
//     M = max_i m_i,  w_i = s_i exp(m_i - M),  out = sum_i w_i o_i / sum_i w_i,
// the running sums rescaled when a later batch raises M. The loads of a batch
// (maxima, sums and the output rows of up to 16 partials) are all issued
// before any of them is used; further output rows follow 16 at a time. All
// reductions run in a fixed order.
template <int D, typename OUT>
__global__ __launch_bounds__(kReduceThreads) void lse_reduce_kernel(ReduceParams p) {
    constexpr int DPL = D / kWave;              // output elements per lane
    constexpr int PRE = 16;                     // partial outputs loaded together
    __shared__ int slots[kReduceThreads / kWave][kWave];
    const int kvh = blockIdx.x;
    const int s = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    const int G = p.group, Hq = p.num_q_heads, NP = p.num_partitions;
    const int L = call_len(p.context_lens[s], p.skip_blocks);
    const bool bad = context_unreadable(L, p.table_blocks, NP, p.partition_blocks, p.num_blocks);
    if (p.extra_count == 0 && (bad || L == 0))
        return;                                // the decode kernel wrote this row
    if (bad) {                                 // cascade: an unreadable suffix
        for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
            const int h = idx / D, d = idx - (idx / D) * D;
            store_out<OUT>(p.out, ((int64_t)s * Hq + kvh * G + h) * D + d, __builtin_nanf(""));
        }
        return;
    }
    const int nblk = (L + kBlockSize - 1) / kBlockSize;
    const int own = (nblk + p.partition_blocks - 1) / p.partition_blocks;   // 0 when L == 0
    if (p.extra_count == 0 && own <= 1)
        return;                                // written directly by its only partition
    const int total = own + p.extra_count;     // partial slots: own partitions, then extras
    for (int h = wave; h < G; h += nw) {
        const int64_t row = (int64_t)s * Hq + (int64_t)kvh * G + h;
        const int64_t base = row * p.part_stride;
        float M = -INFINITY, T = 0.0f;
        float acc[DPL];
#pragma unroll
        for (int e = 0; e < DPL; ++e)
            acc[e] = 0.0f;
        for (int c0 = 0; c0 < total; c0 += kWave) {
            const int i = c0 + lane;
            const int n = min(kWave, total - c0);
            slots[wave][lane] = i < own ? i : p.extra_base + (i - own);
            wave_lds_sync();
            // Lane j < n holds partial j's statistics; the first PRE outputs are
            // requested together with them.
            const int my = lane < n ? slots[wave][lane] : 0;
            const float mv = lane < n ? p.part_max[base + my] : -INFINITY;
            const float sv = lane < n ? p.part_sum[base + my] : 0.0f;
            float ov[PRE][DPL];
#pragma unroll
            for (int j = 0; j < PRE; ++j) {
                // Past the batch's partials the load re-reads slot 0 of the row
                // (always inside the workspace); the value is not used.
                const int sj = j < n ? slots[wave][j] : 0;
                const float* po = p.part_out + (base + sj) * D + lane;
#pragma unroll
                for (int e = 0; e < DPL; ++e)
                    ov[j][e] = po[e * kWave];
            }
            float cm = mv;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1)
                cm = fmaxf(cm, __shfl_xor(cm, o, kWave));
            const float Mn = fmaxf(M, cm);
            const float scale = M == Mn ? 1.0f : __builtin_amdgcn_exp2f((M - Mn) * kLog2e);
            const float wv = lane < n ? sv * __builtin_amdgcn_exp2f((mv - Mn) * kLog2e) : 0.0f;
            float ws = wv;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1)
                ws += __shfl_xor(ws, o, kWave);
            T = T * scale + ws;
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                acc[e] *= scale;
#pragma unroll
            for (int j = 0; j < PRE; ++j) {
                if (j < n) {
                    const float w = readlane_f(wv, j);
#pragma unroll
                    for (int e = 0; e < DPL; ++e)
                        acc[e] = fmaf(w, ov[j][e], acc[e]);
                }
            }
            // The batch's remaining partials, PRE at a time, each group's
            // loads in flight together.
            for (int j0 = PRE; j0 < n; j0 += PRE) {
#pragma unroll
                for (int j = 0; j < PRE; ++j) {
                    const int sj = j0 + j < n ? slots[wave][j0 + j] : 0;
                    const float* po = p.part_out + (base + sj) * D + lane;
#pragma unroll
                    for (int e = 0; e < DPL; ++e)
                        ov[j][e] = po[e * kWave];
                }
#pragma unroll
                for (int j = 0; j < PRE; ++j) {
                    if (j0 + j < n) {
                        const float w = readlane_f(wv, j0 + j);
#pragma unroll
                        for (int e = 0; e < DPL; ++e)
                            acc[e] = fmaf(w, ov[j][e], acc[e]);
                    }
                }
            }
            M = Mn;
            wave_lds_sync();
        }
#pragma unroll
        for (int e = 0; e < DPL; ++e)
            store_out<OUT>(p.out, row * D + lane + e * kWave, acc[e] / T);
    }
}

template <typename KV, int D, int GMAX, typename OUT>
hipError_t launch_decode_grid(const DecodeParams& p, int num_seqs, int grid_partitions, int waves,
                              hipStream_t stream) {
    const size_t lds = decode_lds_bytes(KV::kBytes, D, p.group, waves);
    hipLaunchKernelGGL((paged_decode_kernel<KV, D, GMAX, OUT>),
                       dim3(p.num_kv_heads, num_seqs, grid_partitions), dim3(waves * kWave), lds,
                       stream, p);
    return hipGetLastError();
}

template <typename KV, int D, int GMAX, typename OUT>
hipError_t launch_decode_t(const DecodeParams& p, int num_seqs, int grid_partitions, int waves,
                           hipStream_t stream) {
    if (!p.persistent)
        return launch_decode_grid<KV, D, GMAX, OUT>(p, num_seqs, grid_partitions, waves, stream);
    const auto kernel = paged_decode_persistent_kernel<KV, D, GMAX, OUT>;
    // Persistent: as many workgroups as the GPU keeps resident at once (never
    // more than there can be items).
    const size_t lds = decode_lds_bytes(KV::kBytes, D, p.group, waves) + persistent_lds_bytes(num_seqs);
    int dev = 0, per_cu = 0;
    DeviceInfo info{};
    hipError_t e = current_device_info(&dev, &info);
    if (e != hipSuccess)
        return e;
    if (lds > static_cast<size_t>(info.max_lds)) {
        // The sequence list does not fit one workgroup's LDS: one workgroup
        // per (KV head, sequence, partition) computes the same partials.
        DecodeParams g = p;
        g.persistent = 0;
        return launch_decode_grid<KV, D, GMAX, OUT>(g, num_seqs, grid_partitions, waves, stream);
    }
    e = resident_workgroups_per_cu(dev, reinterpret_cast<const void*>(kernel), waves * kWave, lds,
                                   &per_cu);
    if (e != hipSuccess)
        return e;
    const int64_t bound = static_cast<int64_t>(num_seqs) * p.num_kv_heads * grid_partitions;
    const int64_t wgs = std::max<int64_t>(1, std::min<int64_t>(bound, static_cast<int64_t>(info.cus) *
                                                                         std::max(per_cu, 1)));
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(wgs)), dim3(waves * kWave), lds, stream, p);
    return hipGetLastError();
}

template <typename KV, int D, typename OUT>
hipError_t launch_decode_g(const DecodeParams& p, int num_seqs, int grid_partitions, int waves,
                           hipStream_t stream) {
    switch (decode_gmax(p.group)) {
    case 1: return launch_decode_t<KV, D, 1, OUT>(p, num_seqs, grid_partitions, waves, stream);
    case 2: return launch_decode_t<KV, D, 2, OUT>(p, num_seqs, grid_partitions, waves, stream);
    case 4: return launch_decode_t<KV, D, 4, OUT>(p, num_seqs, grid_partitions, waves, stream);
    case 8: return launch_decode_t<KV, D, 8, OUT>(p, num_seqs, grid_partitions, waves, stream);
    default: return launch_decode_t<KV, D, 16, OUT>(p, num_seqs, grid_partitions, waves, stream);
    }
}

template <typename KV, int D>
hipError_t launch_decode_o(const DecodeParams& p, int out_bf16, int num_seqs, int grid_partitions,
                           int waves, hipStream_t stream) {
    return out_bf16 ? launch_decode_g<KV, D, BF16>(p, num_seqs, grid_partitions, waves, stream)
                    : launch_decode_g<KV, D, F32>(p, num_seqs, grid_partitions, waves, stream);
}

}  // namespace

hipError_t launch_reduce(const ReduceParams& p, int head_size, int out_bf16, int num_seqs,
                         hipStream_t stream) {
    const dim3 grid(p.num_kv_heads, num_seqs);
    if (head_size == 64) {
        if (out_bf16)
            hipLaunchKernelGGL((lse_reduce_kernel<64, BF16>), grid, dim3(kReduceThreads), 0, stream, p);
        else
            hipLaunchKernelGGL((lse_reduce_kernel<64, F32>), grid, dim3(kReduceThreads), 0, stream, p);
    } else {
        if (out_bf16)
            hipLaunchKernelGGL((lse_reduce_kernel<128, BF16>), grid, dim3(kReduceThreads), 0, stream, p);
        else
            hipLaunchKernelGGL((lse_reduce_kernel<128, F32>), grid, dim3(kReduceThreads), 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int kv_bf16, int head_size, int out_bf16,
                         int num_seqs, int grid_partitions, int waves, hipStream_t stream) {
    if (kv_bf16) {
        return head_size == 64
                   ? launch_decode_o<BF16, 64>(p, out_bf16, num_seqs, grid_partitions, waves, stream)
                   : launch_decode_o<BF16, 128>(p, out_bf16, num_seqs, grid_partitions, waves, stream);
    }
    return head_size == 64
               ? launch_decode_o<F32, 64>(p, out_bf16, num_seqs, grid_partitions, waves, stream)
               : launch_decode_o<F32, 128>(p, out_bf16, num_seqs, grid_partitions, waves, stream);
}

}  // namespace pa

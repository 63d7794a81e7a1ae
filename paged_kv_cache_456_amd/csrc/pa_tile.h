// pa_tile.h -- the step shared by the MFMA tile kernels (the shared-prefix
// kernel of pa_cascade.hip and the multi-token-query kernel of
// pa_prefill.hip): a workgroup of NW waves, each wave holding RT tiles of 16
// query rows of one KV head, streams 32 context tokens (two 16-token blocks)
// per step and keeps a running softmax per row.
//
// What is computed is standard scaled dot-product attention over the tokens
// a row may see (the pages print no formula), with the online max/sum
// rescaling that lets the context be consumed in pieces.
//
// Layouts (v_mfma_f32_16x16x32_bf16; lane l = 16 g + r16):
//   * Q^T K is computed as K Q^T: A = K (lane: token r16 of a block, 16-byte
//     chunks g + 4c of its row, read from LDS), B = Q (lane: row r16, the
//     same chunks). The result gives lane l the logits of row r16 for tokens
//     4g + j (first block) and 16 + 4g + j (second block), j < 4, so each
//     row's statistics live in the four lanes r16 + 16 g: the row max is an
//     in-lane max over 8 values and two row swaps, and m, the
//     sum and the rescale factor are one value per lane.
//   * P V is computed as V^T P^T with the MFMA's 32 k slots mapped to the
//     step's tokens as slot 8g + i -> token 4g + i (i < 4) and 16 + 4g + i - 4
//     (i >= 4): B = P^T is then exactly the 8 P values lane l already holds
//     (no exchange, no LDS round trip), and A = V^T (row d, those 8 tokens)
//     is two 8-byte reads of the transposed V rows in LDS. The output tile
//     gives lane l the values of row r16 at columns 16 n + 4 g + j.
//   * P enters the MFMA split into a bf16 high part and a bf16 remainder
//     (two MFMAs), which keeps about 16 bits of P.
//   * K sits in LDS with each row's 16-byte chunks XOR-swizzled by the token
//     (chunk j of token t at slot j ^ (t mod CH)), so that the A-operand
//     reads (16 tokens, one chunk) hit 16 different banks; V^T rows are
//     padded to kVtStride bf16.
#pragma once

#include "pa_device.h"

namespace pa {
namespace tile {

using dev::bf16x8;
using dev::f32x4;
using dev::u16x8;
using dev::u32x4;

constexpr int kStepTokens = 32;                 // two blocks per step
constexpr float kSlack = 8.0f;                  // base-2 headroom of a row's reference max
constexpr int kVtStride = kStepTokens + 8;      // bf16 per transposed V row (80 bytes)

template <int D, int NW>
struct Shape {
    static constexpr int ROW = D * 2;                     // bytes per token row (bf16)
    static constexpr int TILE = kBlockSize * ROW;         // bytes per (block, head) tile
    static constexpr int CH = ROW / 16;                   // 16-byte chunks per row
    static constexpr int NQ = CH / 4;                     // K chunks per lane per block
    static constexpr int NT = D / 16;                     // 16-column output tiles
    static constexpr int THREADS = NW * kWave;
    static constexpr int KITEMS = kStepTokens * CH;       // 16-byte K chunks of a step
    static constexpr int KPT = KITEMS / THREADS;          // K chunks per thread
    static constexpr int VITEMS = (kStepTokens / 2) * CH; // (token pair, chunk) items of a step
    static_assert(KPT >= 1 && KITEMS % THREADS == 0, "whole K chunks per thread");
    static_assert(VITEMS <= THREADS && THREADS % VITEMS == 0, "one V item per thread");
};

// LDS of the step: K and V^T, two buffers each, used on alternate steps (a
// buffer is written again two steps later, after a barrier that every wave
// passes only once done with it).
template <int D, int NW>
struct Lds {
    u32x4 k[2][Shape<D, NW>::KITEMS];
    uint16_t vt[2][D][kVtStride];
};

// This thread's share of a step's loads: KPT 16-byte K chunks and one V pair
// (two adjacent tokens of one 16-byte chunk). The loads of a step are issued
// one step ahead and written to LDS (K swizzled, V transposed) when the step
// starts.
template <int D, int NW>
struct StepData {
    u32x4 kq[Shape<D, NW>::KPT], vr[2];
};

template <int D, int NW>
struct Loader {
    using S = Shape<D, NW>;
    int kslot[S::KPT], koff[S::KPT], kblk[S::KPT];
    int tp, vc, vblk, voff;

    __device__ __forceinline__ void init() {
#pragma unroll
        for (int k = 0; k < S::KPT; ++k) {
            const int q = threadIdx.x + k * S::THREADS;      // chunk q % CH of token q / CH
            const int t = q / S::CH, j = q % S::CH;
            kslot[k] = t * S::CH + (j ^ (t & (S::CH - 1)));
            kblk[k] = t >> 4;
            koff[k] = (t & 15) * S::ROW + j * 16;
        }
        const int vi = threadIdx.x % S::VITEMS;
        tp = vi % (kStepTokens / 2);
        vc = vi / (kStepTokens / 2);
        vblk = tp >> 3;
        voff = (2 * tp - 16 * vblk) * S::ROW + vc * 16;
    }

    // The step's two blocks id0, id1 (a lone last block passes id1 = id0).
    __device__ __forceinline__ void load(StepData<D, NW>& d, const char* kbase, const char* vbase,
                                         int64_t blk_stride, int id0, int id1) const {
#pragma unroll
        for (int k = 0; k < S::KPT; ++k)
            d.kq[k] = *reinterpret_cast<const u32x4*>(kbase + (int64_t)(kblk[k] ? id1 : id0) * blk_stride +
                                                      koff[k]);
        const char* v = vbase + (int64_t)(vblk ? id1 : id0) * blk_stride + voff;
        d.vr[0] = *reinterpret_cast<const u32x4*>(v);
        d.vr[1] = *reinterpret_cast<const u32x4*>(v + S::ROW);
    }

    // Writes a loaded step to LDS buffer `buf`; V of step tokens >= vis_end
    // is written as zeros (block tails may hold anything, even NaN, and must
    // contribute exactly nothing to P V).
    __device__ __forceinline__ void stage(const StepData<D, NW>& d, Lds<D, NW>& l, int buf,
                                          int vis_end) const {
#pragma unroll
        for (int k = 0; k < S::KPT; ++k)
            l.k[buf][kslot[k]] = d.kq[k];
        const bool za = 2 * tp >= vis_end, zb = 2 * tp + 1 >= vis_end;
        uint32_t* col = reinterpret_cast<uint32_t*>(&l.vt[buf][vc * 8][2 * tp]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t a = za ? 0u : d.vr[0][e], b = zb ? 0u : d.vr[1][e];
            col[(2 * e) * (kVtStride / 2)] = (a & 0xFFFFu) | (b << 16);
            col[(2 * e + 1) * (kVtStride / 2)] = (a >> 16) | (b & 0xFFFF0000u);
        }
    }
};

// Runs steps 0 .. nsteps - 1: step st is staged from the StepData into LDS
// buffer st % 2, the loads of step st + 1 go out into the StepData (clamped
// to the last step, so that no load sits under a branch) and land while the
// step computes, a workgroup barrier, then compute(st, buf). load(d, st)
// issues step st's loads, stage(d, st, buf) writes them to LDS.
template <int D, int NW, typename LoadFn, typename StageFn, typename ComputeFn>
__device__ __forceinline__ void run_steps(int nsteps, LoadFn load, StageFn stage, ComputeFn compute) {
    StepData<D, NW> d;
    load(d, 0);
#pragma nounroll
    for (int st = 0; st < nsteps; ++st) {
        const int buf = st & 1;
        stage(d, st, buf);
        load(d, min(st + 1, nsteps - 1));
        dev::lds_barrier();                 // the step's K and V^T are in LDS
        compute(st, buf);
    }
}

// Running state of a wave's RT row tiles: the reference maximum m (base 2;
// every logit seen is at most m + kSlack) and the partial sum of
// 2^(logit - m) over lane l's tokens for row r16 of each tile, and the output
// tiles (lane l: row r16, columns 16 n + 4 g + j).
template <int D, int RT>
struct RowState {
    float m[RT], lsum[RT];
    f32x4 o[RT][D / 16];

    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            m[t] = -INFINITY;
            lsum[t] = 0.0f;
#pragma unroll
            for (int n = 0; n < D / 16; ++n)
                o[t][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }

    // Row sum of tile t (every lane of the row's four), over the same row
    // swaps as row_group_max.
    __device__ __forceinline__ float row_sum(int t) const {
        const uint32_t u = __float_as_uint(lsum[t]);
        const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        const float h = __uint_as_float(a[0]) + __uint_as_float(a[1]);
        const uint32_t w = __float_as_uint(h);
        const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
        return __uint_as_float(b[0]) + __uint_as_float(b[1]);
    }
};

// Maximum over the four lanes r16, r16 + 16, r16 + 32, r16 + 48 that hold one
// row's values, returned to all four: gfx950's row swaps exchange 16-lane
// rows (and 32-lane halves) between two registers in the VALU, with no LDS
// round trip. Called with the same value as both operands, each lane gets
// its own value and its partner's (lane ^ 16, then lane ^ 32).
__device__ __forceinline__ float row_group_max(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t w = __float_as_uint(m);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// P as the B operand, split into bf16 high parts and bf16 remainders, two
// values per 32-bit word (k slots 2i, 2i + 1 in word i).
__device__ __forceinline__ void split_p(const float (&v)[8], u32x4& hi, u32x4& lo) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16x2 h = {static_cast<__bf16>(v[2 * i]), static_cast<__bf16>(v[2 * i + 1])};
        const uint32_t hb = __builtin_bit_cast(uint32_t, h);
        const float h0 = __uint_as_float(hb << 16), h1 = __uint_as_float(hb & 0xFFFF0000u);
        const bf16x2 r = {static_cast<__bf16>(v[2 * i] - h0), static_cast<__bf16>(v[2 * i + 1] - h1)};
        hi[i] = hb;
        lo[i] = __builtin_bit_cast(uint32_t, r);
    }
}

// One step for a wave: logits of its RT tiles against the 32 tokens in LDS
// buffer `buf`, online softmax, and P V into the output tiles.
// visible(t, tok) says whether row r16 of tile t sees step token tok (hidden
// logits are dropped by select, never scaled); full(t), the same for every
// lane of the wave, says that every row of tile t sees all 32 tokens, and
// skips the selects. The output tiles are rescaled only when some row's
// reference maximum moves (see kSlack).
// Order: the K Q^T products of every tile and the V^T reads go out first;
// then tile by tile the softmax (VALU) runs while the matrix core still works
// on earlier products, and the tile's P V products are issued behind it.
template <int D, int NW, int RT, typename Visible, typename Full>
__device__ __forceinline__ void attend(const Lds<D, NW>& l, int buf, const u32x4 (&qa)[RT][Shape<D, NW>::NQ],
                                       float scale_log2, Visible visible, Full full, RowState<D, RT>& st) {
    using S = Shape<D, NW>;
    constexpr int NQ = S::NQ, CH = S::CH, NT = S::NT;
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane >> 4, r16 = lane & 15;
    // K as the A operand: token r16 of each block, chunks g + 4c.
    u32x4 k0[NQ], k1[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
        const int cc = g + 4 * c;
        k0[c] = l.k[buf][r16 * CH + (cc ^ (r16 & (CH - 1)))];
        k1[c] = l.k[buf][(16 + r16) * CH + (cc ^ ((16 + r16) & (CH - 1)))];
    }
    f32x4 a0[RT], a1[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        a0[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        a1[t] = a0[t];
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            a0[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k0[c]),
                                                            __builtin_bit_cast(bf16x8, qa[t][c]), a0[t], 0, 0, 0);
            a1[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k1[c]),
                                                            __builtin_bit_cast(bf16x8, qa[t][c]), a1[t], 0, 0, 0);
        }
    }
    // V^T as the A operand: row 16 n + r16, tokens 4g .. 4g+3 and 16 + 4g .. 16 + 4g + 3.
    u32x4 va[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const uint16_t* vrow = &l.vt[buf][n * 16 + r16][0];
        const uint2 lo4 = *reinterpret_cast<const uint2*>(vrow + 4 * g);
        const uint2 hi4 = *reinterpret_cast<const uint2*>(vrow + 16 + 4 * g);
        va[n] = u32x4{lo4.x, lo4.y, hi4.x, hi4.y};
    }
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[j] = a0[t][j] * scale_log2;
            x[4 + j] = a1[t][j] * scale_log2;
        }
        if (!full(t)) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[j] = visible(t, 4 * g + j) ? x[j] : -INFINITY;
                x[4 + j] = visible(t, 16 + 4 * g + j) ? x[4 + j] : -INFINITY;
            }
        }
        float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                         fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        mx = row_group_max(mx);
        // The row's reference m moves only when a logit exceeds it by more
        // than kSlack (P then stays <= 2^kSlack; P, the sum and the output
        // share the reference, so the result is the same in exact arithmetic)
        // and the output tiles are rescaled only then.
        const bool grow = mx > st.m[t] + kSlack;
        const float mn = grow ? mx : st.m[t];
        // A row that has seen nothing yet (mn = -inf) keeps a zero state.
        const float alpha = grow ? __builtin_amdgcn_exp2f(st.m[t] - mn) : 1.0f;
        float pv[8];
        float ps = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            pv[i] = mn == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x[i] - mn);
            ps += pv[i];
        }
        st.lsum[t] = st.lsum[t] * alpha + ps;
        st.m[t] = mn;
        if (__ballot(grow) != 0) {
#pragma unroll
            for (int n = 0; n < NT; ++n)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    st.o[t][n][j] *= alpha;
        }
        u32x4 phi, plo;
        split_p(pv, phi, plo);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            st.o[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va[n]),
                                                                 __builtin_bit_cast(bf16x8, phi), st.o[t][n], 0, 0, 0);
            st.o[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va[n]),
                                                                 __builtin_bit_cast(bf16x8, plo), st.o[t][n], 0, 0, 0);
        }
    }
}

}  // namespace tile
}  // namespace pa

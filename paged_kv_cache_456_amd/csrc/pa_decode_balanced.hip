// pa_decode_balanced.hip -- work-balanced paged decode attention for gfx950,
// optionally fused with the step's cache write.
//
// What is computed is the decode of pa_decode.hip: each sequence's new query
// token attends over its context, read from 16-token blocks scattered through
// the pool and reached through its block table ("Idea 1: PagedAttention" on
// the day-9 post; "The idea vLLM started from: pages" on "What vLLM Is and
// Why It Exists"). With the write fused, each sequence's new key and value
// vectors are first stored at position L - 1 of its context (the slot its
// table gives that position), as the cache write does, and attended to with
// the rest ("The problem a naive server has", point 3: every produced token's
// K/V is kept and reused).
//
// Schedule. The decode is bandwidth-bound and contexts differ widely in
// length, so the work is split by bytes, not by sequence. A unit is one
// 16-token block of one (sequence, KV head) row; the units of all rows form a
// line, rows in (sequence, KV head) order and blocks in order within a row (a
// row with nothing to read counts one unit, which writes its zero or NaN
// row). The line is cut into equal contiguous ranges, one per resident
// workgroup, and each workgroup's range into equal contiguous ranges, one per
// wave. A wave streams its range on its own (no barrier): a row that lies
// wholly inside the range is finished and written by the wave; the first and
// last row of the range, when cut, leave their online-softmax state in LDS.
// At the end (one barrier) the workgroup merges the states of each row cut
// between its waves, in wave order; a row that lies wholly inside the
// workgroup is written, and the at most two rows cut by the workgroup's own
// boundaries become partials (max, sum, normalised output) in the workspace,
// with a descriptor that the small combining kernel below uses to merge them
// in workgroup order. Every merge runs in a fixed order that depends only on
// the context lengths and the grid, never on where the blocks sit in the
// pool.
#include <algorithm>
#include <type_traits>

#include "pa_decode_core.h"

namespace pa {
namespace {

using namespace core;

// Units of a row (one per block; one for a row with nothing to read).
__device__ __forceinline__ int row_units(int L, const DecodeParams& p) {
    if (L == 0 || context_unreadable(L, p.max_blocks_per_seq, 1, p.max_blocks_per_seq, p.num_blocks))
        return 1;
    return (L + kBlockSize - 1) / kBlockSize;
}

// LDS layout (floats unless noted), NW waves:
//   ptile  [NW][BPW * 16][GP]            P tiles of the rounds (pa_decode_core.h)
//   pieces [2 NW][2 GP + GMAX * D]       per-wave cut-row states: m (base 2),
//                                        sum, unnormalised o
//   prow   [2 NW] int                    row id of each piece, -1 for none
//   start  [S + 1] int                   first unit of each sequence
template <typename KV, int D, int GMAX>
struct BalancedLayout {
    static constexpr int BPW = decode_bpw(KV::kBytes, D, GMAX);
    static constexpr int GP = decode_pstride(GMAX);
    static constexpr int kTile = BPW * kBlockSize * GP;          // P tile floats per wave
    static constexpr int kPiece = 2 * GP + GMAX * D;             // floats per piece
};

template <typename KV, int D, int GMAX>
size_t balanced_lds_bytes(int waves, int num_seqs) {
    using Ly = BalancedLayout<KV, D, GMAX>;
    return sizeof(float) * (static_cast<size_t>(waves) * Ly::kTile + 2 * static_cast<size_t>(waves) * Ly::kPiece) +
           sizeof(int) * (2 * static_cast<size_t>(waves) + static_cast<size_t>(num_seqs) + 1);
}

// Writes the final output of row (s, kvh) from one wave's totals: heads
// h < G, out = o / sum (lanes of the first token row write their chunk).
template <typename KV, int D, int GMAX, typename OUT>
__device__ __forceinline__ void write_row(const DecodeParams& p, int s, int kvh,
                                          const WaveAcc<KV, D, GMAX>& acc, const float (&srow)[4]) {
    using Gm = Geometry<KV, D>;
    constexpr int CH = Gm::kCh, EPC = Gm::kEpc;
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
        if (h >= p.group)
            break;
        const float S = readlane_f(srow[h & 3], 16 * (h >> 2));
        if (lane < CH) {
            const int64_t base = ((int64_t)s * p.num_q_heads + (int64_t)kvh * p.group + h) * D + lane * EPC;
#pragma unroll
            for (int e = 0; e < EPC; ++e)
                store_out<OUT>(p.out, base + e, acc.o[h][e] / S);
        }
    }
}

// Stores one wave's totals as piece `slot` of the workgroup's LDS.
template <typename KV, int D, int GMAX>
__device__ __forceinline__ void store_piece(float* piece, int* prow, int slot, int row,
                                            const WaveAcc<KV, D, GMAX>& acc, const float (&srow)[4]) {
    using Gm = Geometry<KV, D>;
    using Ly = BalancedLayout<KV, D, GMAX>;
    constexpr int CH = Gm::kCh, EPC = Gm::kEpc, GP = Ly::GP;
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane >> 4, r16 = lane & 15;
    float* pc = piece + slot * Ly::kPiece;
    if (r16 == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int h = 4 * g + j;
            if (h < GMAX) {
                pc[h] = acc.m[j];
                pc[GP + h] = srow[j];
            }
        }
    }
    if (lane < CH) {
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
            float* dst = pc + 2 * GP + h * D + lane * EPC;
#pragma unroll
            for (int e = 0; e < EPC; e += 4)
                *reinterpret_cast<f32x4*>(dst + e) =
                    f32x4{acc.o[h][e], acc.o[h][e + 1], acc.o[h][e + 2], acc.o[h][e + 3]};
        }
    }
    if (lane == 0)
        prow[slot] = row;
}

// Last sequence whose first unit is <= u (start[0] = 0 <= u < start[S]).
__device__ __forceinline__ int seq_of_unit(const int* start, int S, int u) {
    int lo = 0, hi = S;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (start[mid] <= u)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

// First unit of workgroup w's range when U units are split over n workgroups.
__device__ __forceinline__ int range_start(int64_t U, int w, int n) {
    return static_cast<int>(U * w / n);
}

template <typename KV, int D, int GMAX>
constexpr int balanced_waves_per_simd() {
    return (GMAX <= 4 && D * KV::kBytes <= 256) ? 3 : 2;
}

template <typename KV, int D, int GMAX, typename OUT, bool WRITE>
__global__ __launch_bounds__(kBalancedWaves * kWave)
__attribute__((amdgpu_waves_per_eu(balanced_waves_per_simd<KV, D, GMAX>())))
void paged_decode_balanced_kernel(BalancedParams bp) {
    using Gm = Geometry<KV, D>;
    using Ly = BalancedLayout<KV, D, GMAX>;
    constexpr int BPW = Ly::BPW, GP = Ly::GP, ROW = Gm::kRow, CH = Gm::kCh;
    (void)ROW;
    (void)CH;
    extern __shared__ float smem[];
    const DecodeParams& p = bp.d;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nw = blockDim.x / kWave;
    const int S = p.num_seqs, Hkv = p.num_kv_heads, G = p.group;
    float* ptile = smem + wave * Ly::kTile;
    float* pieces = smem + nw * Ly::kTile;
    int* prow = reinterpret_cast<int*>(pieces + 2 * nw * Ly::kPiece);
    int* start = prow + 2 * nw;

    // First unit of every sequence (exclusive prefix sum of units * Hkv).
    if (wave == 0) {
        int carry = 0;
        for (int c0 = 0; c0 < S; c0 += kWave) {
            const int i = c0 + lane;
            const int v = i < S ? row_units(p.context_lens[i], p) * Hkv : 0;
            int incl = v;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const int t = __shfl_up(incl, off, kWave);
                if (lane >= off)
                    incl += t;
            }
            if (i < S)
                start[i] = carry + incl - v;
            carry += __shfl(incl, kWave - 1, kWave);
        }
        if (lane == 0)
            start[S] = carry;
    }
    if (threadIdx.x < 2 * nw)
        prow[threadIdx.x] = -1;
    __syncthreads();

    const int U = __builtin_amdgcn_readfirstlane(start[S]);
    // Workgroups past the unit count get no range: every range is non-empty.
    const int nwg = min(static_cast<int>(gridDim.x), U);
    const int w = blockIdx.x;
    const int ua = w < nwg ? range_start(U, w, nwg) : 0;
    const int ub = w < nwg ? range_start(U, w + 1, nwg) : 0;
    const int u0 = ua + static_cast<int>(static_cast<int64_t>(ub - ua) * wave / nw);
    const int u1 = ua + static_cast<int>(static_cast<int64_t>(ub - ua) * (wave + 1) / nw);

    // ---- this wave's range, row segment by row segment
    int u = u0;
    while (u < u1) {
        const int s = __builtin_amdgcn_readfirstlane(seq_of_unit(start, S, u));
        const int s0 = __builtin_amdgcn_readfirstlane(start[s]);
        const int nb = (__builtin_amdgcn_readfirstlane(start[s + 1]) - s0) / Hkv;   // units per row
        const int rem = u - s0;
        const int kvh = rem / nb;
        const int j0 = rem - kvh * nb;
        const int j1 = min(nb, j0 + (u1 - u));
        const int row = s * Hkv + kvh;
        const int L = p.context_lens[s];
        const bool whole = j0 == 0 && j1 == nb;
        const bool bad = context_unreadable(L, p.max_blocks_per_seq, 1, p.max_blocks_per_seq,
                                            p.num_blocks);
        if (bad || L == 0) {
            // One unit, the whole row: a zero row (empty) or a NaN row (unreadable).
            const float v = bad ? __builtin_nanf("") : 0.0f;
            for (int i = lane; i < G * D; i += kWave)
                store_out<OUT>(p.out, ((int64_t)s * p.num_q_heads + (int64_t)kvh * G) * D + i, v);
        } else {
            u32x4 qa[Gm::kNq];
            load_query<KV, D>(p, kvh, s, qa);
            // With the write fused, the segment that ends the row streams only
            // the tokens before the new one; the new token's K and V come from
            // the inputs (the slot being written is never read), loaded before
            // the blocks are streamed.
            const bool with_new = WRITE && j1 == nb;
            NewToken<KV, D> tok;
            if constexpr (WRITE) {
                if (with_new) {
                    const int64_t src = ((int64_t)s * Hkv + kvh) * ROW;
                    tok = load_new_token<KV, D>(static_cast<const char*>(bp.new_key) + src,
                                                static_cast<const char*>(bp.new_value) + src);
                }
            }
            WaveAcc<KV, D, GMAX> acc;
            acc.reset();
            const int L_old = with_new ? L - 1 : L;
            const int pb1 = min(j1, (L_old + kBlockSize - 1) / kBlockSize);
            if (pb1 > j0)
                accumulate_blocks<KV, D, GMAX>(p, ptile, qa, kvh, s, L_old, pb1, j0, BPW,
                                               (pb1 - j0 + BPW - 1) / BPW, acc);
            if constexpr (WRITE) {
                if (with_new) {
                    accumulate_token<KV, D, GMAX>(p, qa, tok, acc);
                    store_new_token<KV, D>(p, tok, s, kvh, L, 0);
                }
            }
            float srow[4];
            wave_totals<KV, D, GMAX>(acc, srow);
            if (whole)
                write_row<KV, D, GMAX, OUT>(p, s, kvh, acc, srow);
            else
                store_piece<KV, D, GMAX>(pieces, prow, 2 * wave + (u == u0 ? 0 : 1), row, acc, srow);
        }
        u += j1 - j0;
    }
    __syncthreads();
    if (ua >= ub) {
        if (threadIdx.x == 0)
            bp.desc[w] = int4{-1, 0, 0, 0};
        return;
    }

    // ---- rows cut between waves: merge in wave order; rows cut by this
    // workgroup's own boundaries become partials.
    const int s_first = seq_of_unit(start, S, ua);
    const int nb_first = (start[s_first + 1] - start[s_first]) / Hkv;
    const int row_first = s_first * Hkv + (ua - start[s_first]) / nb_first;
    const int row_first_u0 = start[s_first] + (row_first - s_first * Hkv) * nb_first;
    const int s_last = seq_of_unit(start, S, ub - 1);
    const int nb_last = (start[s_last + 1] - start[s_last]) / Hkv;
    const int row_last = s_last * Hkv + (ub - 1 - start[s_last]) / nb_last;
    const int row_last_u1 = start[s_last] + (row_last - s_last * Hkv + 1) * nb_last;
    const bool first_cut = ua > row_first_u0;
    const bool last_cut = ub < row_last_u1;
    const int slot_first = 2 * w;
    const int slot_last = row_last == row_first ? 2 * w : 2 * w + 1;

    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
        const int h = idx / D;
        const int d = idx - h * D;
        int cur = -1;
        float M = -INFINITY, Ssum = 0.0f, O = 0.0f;
        auto flush = [&]() {
            const int ps = cur / Hkv, pk = cur - ps * Hkv;
            int slot = -1;
            if (cur == row_first && first_cut)
                slot = slot_first;
            else if (cur == row_last && last_cut)
                slot = slot_last;
            if (slot < 0) {
                store_out<OUT>(p.out, ((int64_t)ps * p.num_q_heads + (int64_t)pk * G + h) * D + d, O / Ssum);
            } else {
                const int64_t pi = (int64_t)slot * G + h;
                p.part_out[pi * D + d] = O / Ssum;
                if (d == 0) {
                    p.part_max[pi] = M;
                    p.part_sum[pi] = Ssum;
                }
            }
        };
        for (int i = 0; i < 2 * nw; ++i) {
            const int r = prow[i];
            if (r < 0)
                continue;
            if (r != cur) {
                if (cur >= 0)
                    flush();
                cur = r;
                M = -INFINITY;
                Ssum = 0.0f;
                O = 0.0f;
            }
            const float* pc = pieces + i * Ly::kPiece;
            const float mi = pc[h];
            const float Mn = fmaxf(M, mi);
            const float fo = __builtin_amdgcn_exp2f(M - Mn), fi = __builtin_amdgcn_exp2f(mi - Mn);
            Ssum = Ssum * fo + pc[GP + h] * fi;
            O = O * fo + pc[2 * GP + h * D + d] * fi;
            M = Mn;
        }
        if (cur >= 0)
            flush();
    }

    // Descriptor: this workgroup is the first of the row cut at its end.
    if (threadIdx.x == 0) {
        int4 dsc{-1, 0, 0, 0};
        if (last_cut && !(row_last == row_first && first_cut)) {
            // Last workgroup holding the row's final unit x = row_last_u1 - 1.
            const int64_t x = row_last_u1 - 1;
            const int wb = static_cast<int>(((x + 1) * nwg - 1) / U);
            dsc = int4{row_last, slot_last, wb, 0};
        }
        bp.desc[w] = dsc;
    }
}

// Combines the partials of every row cut between workgroups: row desc.x's
// partial in slot desc.y of workgroup w, then slot 2 w' of each later
// workgroup w' <= desc.z, with log-sum-exp weights (maxima in base 2):
//     M = max_i m_i,  w_i = s_i 2^(m_i - M),  out = sum_i w_i o_i / sum_i w_i.
// One workgroup per descriptor, one wave per query head at a time; the
// statistics of up to 64 partials are loaded together (one lane each) and
// the output rows of up to 16 at a time.
template <int D, typename OUT>
__global__ __launch_bounds__(kReduceThreads) void balanced_reduce_kernel(BalancedParams bp) {
    constexpr int DPL = D / kWave;
    constexpr int PRE = 16;
    const DecodeParams& p = bp.d;
    const int4 dsc = bp.desc[blockIdx.x];
    if (dsc.x < 0)
        return;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    const int G = p.group, Hkv = p.num_kv_heads;
    const int s = dsc.x / Hkv, kvh = dsc.x - (dsc.x / Hkv) * Hkv;
    const int total = dsc.z - static_cast<int>(blockIdx.x) + 1;     // partials of the row
    auto slot_of = [&](int i) { return i == 0 ? dsc.y : 2 * (static_cast<int>(blockIdx.x) + i); };
    for (int h = wave; h < G; h += nw) {
        float M = -INFINITY, T = 0.0f;
        float acc[DPL];
#pragma unroll
        for (int e = 0; e < DPL; ++e)
            acc[e] = 0.0f;
        for (int c0 = 0; c0 < total; c0 += kWave) {
            const int n = min(kWave, total - c0);
            const int64_t my = lane < n ? (int64_t)slot_of(c0 + lane) * G + h : 0;
            const float mv = lane < n ? p.part_max[my] : -INFINITY;
            const float sv = lane < n ? p.part_sum[my] : 0.0f;
            float cm = mv;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1)
                cm = fmaxf(cm, __shfl_xor(cm, o, kWave));
            const float Mn = fmaxf(M, cm);
            const float scale = M == Mn ? 1.0f : __builtin_amdgcn_exp2f(M - Mn);
            const float wv = lane < n ? sv * __builtin_amdgcn_exp2f(mv - Mn) : 0.0f;
            float ws = wv;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1)
                ws += __shfl_xor(ws, o, kWave);
            T = T * scale + ws;
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                acc[e] *= scale;
            for (int j0 = 0; j0 < n; j0 += PRE) {
                float ov[PRE][DPL];
#pragma unroll
                for (int j = 0; j < PRE; ++j) {
                    // Past the batch the load re-reads the row's first partial.
                    const int i = j0 + j < n ? c0 + j0 + j : 0;
                    const float* po = p.part_out + ((int64_t)slot_of(i) * G + h) * D + lane;
#pragma unroll
                    for (int e = 0; e < DPL; ++e)
                        ov[j][e] = po[e * kWave];
                }
#pragma unroll
                for (int j = 0; j < PRE; ++j) {
                    if (j0 + j < n) {
                        const float wj = readlane_f(wv, j0 + j);
#pragma unroll
                        for (int e = 0; e < DPL; ++e)
                            acc[e] = fmaf(wj, ov[j][e], acc[e]);
                    }
                }
            }
            M = Mn;
        }
        const int64_t row = ((int64_t)s * p.num_q_heads + (int64_t)kvh * G + h) * D;
#pragma unroll
        for (int e = 0; e < DPL; ++e)
            store_out<OUT>(p.out, row + lane + e * kWave, acc[e] / T);
    }
}

template <typename KV, int D, int GMAX, typename OUT, bool WRITE>
hipError_t launch_t(const BalancedParams& bp, int max_workgroups, hipStream_t stream) {
    const auto kernel = paged_decode_balanced_kernel<KV, D, GMAX, OUT, WRITE>;
    const size_t lds = balanced_lds_bytes<KV, D, GMAX>(kBalancedWaves, bp.d.num_seqs);
    int dev = 0, per_cu = 0;
    DeviceInfo info{};
    hipError_t e = current_device_info(&dev, &info);
    if (e != hipSuccess)
        return e;
    if (lds > static_cast<size_t>(info.max_lds))
        return hipErrorInvalidValue;
    e = resident_workgroups_per_cu(dev, reinterpret_cast<const void*>(kernel), kBalancedWaves * kWave,
                                   lds, &per_cu);
    if (e != hipSuccess)
        return e;
    const int64_t resident = static_cast<int64_t>(info.cus) * std::max(per_cu, 1);
    const int wgs = static_cast<int>(std::max<int64_t>(
        1, std::min<int64_t>({resident, static_cast<int64_t>(kMaxBalancedWorkgroups),
                              static_cast<int64_t>(max_workgroups)})));
    hipLaunchKernelGGL(kernel, dim3(wgs), dim3(kBalancedWaves * kWave), lds, stream, bp);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((balanced_reduce_kernel<D, OUT>), dim3(wgs), dim3(kReduceThreads), 0, stream, bp);
    return hipGetLastError();
}

template <typename KV, int D, typename OUT, bool WRITE>
hipError_t launch_g(const BalancedParams& bp, int max_workgroups, hipStream_t stream) {
    switch (decode_gmax(bp.d.group)) {
    case 1: return launch_t<KV, D, 1, OUT, WRITE>(bp, max_workgroups, stream);
    case 2: return launch_t<KV, D, 2, OUT, WRITE>(bp, max_workgroups, stream);
    case 4: return launch_t<KV, D, 4, OUT, WRITE>(bp, max_workgroups, stream);
    case 8: return launch_t<KV, D, 8, OUT, WRITE>(bp, max_workgroups, stream);
    default: return launch_t<KV, D, 16, OUT, WRITE>(bp, max_workgroups, stream);
    }
}

template <typename KV, int D, bool WRITE>
hipError_t launch_o(const BalancedParams& bp, int out_bf16, int max_workgroups, hipStream_t stream) {
    return out_bf16 ? launch_g<KV, D, BF16, WRITE>(bp, max_workgroups, stream)
                    : launch_g<KV, D, F32, WRITE>(bp, max_workgroups, stream);
}

template <typename KV, int D>
hipError_t launch_w(const BalancedParams& bp, int out_bf16, int max_workgroups, hipStream_t stream) {
    return bp.new_key ? launch_o<KV, D, true>(bp, out_bf16, max_workgroups, stream)
                      : launch_o<KV, D, false>(bp, out_bf16, max_workgroups, stream);
}

}  // namespace

size_t balanced_lds_bytes_for(int kv_bf16, int head_size, int group, int num_seqs) {
    const int gm = decode_gmax(group);
    auto pick = [&](auto kv, auto d) -> size_t {
        using KV = decltype(kv);
        constexpr int D = decltype(d)::value;
        switch (gm) {
        case 1: return balanced_lds_bytes<KV, D, 1>(kBalancedWaves, num_seqs);
        case 2: return balanced_lds_bytes<KV, D, 2>(kBalancedWaves, num_seqs);
        case 4: return balanced_lds_bytes<KV, D, 4>(kBalancedWaves, num_seqs);
        case 8: return balanced_lds_bytes<KV, D, 8>(kBalancedWaves, num_seqs);
        default: return balanced_lds_bytes<KV, D, 16>(kBalancedWaves, num_seqs);
        }
    };
    if (kv_bf16)
        return head_size == 64 ? pick(BF16{}, std::integral_constant<int, 64>{})
                               : pick(BF16{}, std::integral_constant<int, 128>{});
    return head_size == 64 ? pick(F32{}, std::integral_constant<int, 64>{})
                           : pick(F32{}, std::integral_constant<int, 128>{});
}

hipError_t launch_decode_balanced(const BalancedParams& bp, int kv_bf16, int head_size, int out_bf16,
                                  int max_workgroups, hipStream_t stream) {
    if (kv_bf16)
        return head_size == 64 ? launch_w<BF16, 64>(bp, out_bf16, max_workgroups, stream)
                               : launch_w<BF16, 128>(bp, out_bf16, max_workgroups, stream);
    return head_size == 64 ? launch_w<F32, 64>(bp, out_bf16, max_workgroups, stream)
                           : launch_w<F32, 128>(bp, out_bf16, max_workgroups, stream);
}

}  // namespace pa

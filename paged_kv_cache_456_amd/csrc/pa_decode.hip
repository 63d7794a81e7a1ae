// pa_decode.hip -- paged decode attention kernels for gfx950 (CDNA4).
//
// What is computed: for each sequence, its one new query token attends over
// a KV cache held in 16-token blocks scattered through a shared pool and
// reached through the sequence's block table ("Idea 1: PagedAttention" on
// the day-9 post of skandtandon.pages.dev; "The idea vLLM started from:
// pages" on "What vLLM Is and Why It Exists"). The attention is standard
// scaled dot-product softmax attention (the pages print no formula).
//
// Work decomposition. One workgroup per (KV head, sequence, context
// partition); its waves take the partition's blocks round-robin. Every query
// head of the group that shares the KV head is handled by the same wave, so
// each K/V byte is read from HBM once per step.
//
// Per block (16 tokens x D of one KV head, one contiguous tile):
//   * the physical block id comes from a per-wave register that holds the
//     wave's whole slice of the block table (one vector load per 64 blocks,
//     v_readlane per block): the table is resolved once per wavefront;
//   * K is loaded so that lane l holds token l%16, 16-byte chunks l/16+4c of
//     its row, which is the B-operand layout of a 16x16 MFMA. Q^T K for the
//     whole head group is one MFMA chain (bf16: v_mfma_f32_16x16x32_bf16,
//     fp32: v_mfma_f32_16x16x4_f32), heads as rows, tokens as columns;
//   * softmax statistics are kept online (running max and sum, base-2
//     exponent with scale*log2(e) folded in); the block max is a 16-lane DPP
//     row reduction;
//   * V is loaded fully coalesced (consecutive lanes read consecutive 16-byte
//     chunks); P.V runs on the VALU in fp32 with P in fp32, because P in bf16
//     would cost about 2e-3 of accuracy. P moves from the MFMA layout to the V
//     layout through 1 KB of LDS per wave;
//   * the next block's K and V are prefetched into registers while the
//     current block is computed.
// Waves then merge their (max, sum, output) through LDS in a fixed order, so
// results depend only on logical token positions, never on where the blocks
// sit in the pool.
#include "pa_internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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
    static constexpr int kEpc = 8;   // elements per 16-byte chunk
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
    static constexpr int kEpc = 4;
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

template <typename KV, int D>
struct Tile {
    u32x4 k[Geometry<KV, D>::kNq];
    u32x4 v[Geometry<KV, D>::kNv];
};

// Dynamic LDS layout per workgroup of nw waves:
//   p_lds  [nw][16][16]   P of the current block, [token][head]
//   red_m  [nw][GP]       per-wave running max (base-2 units), GP = GMAX rounded up to 4
//   red_s  [nw][GP]       per-wave sum of exponentials
//   red_o  [nw][GMAX][D]  per-wave unnormalised output
// (GMAX rounded up to 4 keeps red_o 16-byte aligned.)
template <int GMAX>
constexpr int padded_group() { return (GMAX + 3) & ~3; }

template <int GMAX, int D>
__host__ __device__ constexpr size_t decode_lds_bytes(int nw) {
    return sizeof(float) * static_cast<size_t>(nw) * (256 + 2 * padded_group<GMAX>() + GMAX * D);
}

template <typename KV, int D, int GMAX, typename OUT>
__global__ __launch_bounds__(kMaxWaves * kWave) void paged_decode_kernel(DecodeParams p) {
    using Gm = Geometry<KV, D>;
    using Op = Ops<KV>;
    constexpr int NQ = Gm::kNq, NV = Gm::kNv, CH = Gm::kCh, TPL = Gm::kTpl, EPC = Gm::kEpc;
    constexpr int ROW = Gm::kRow, TILE = Gm::kTile;

    extern __shared__ float smem[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    const int kvh = blockIdx.x;
    const int s = blockIdx.y;
    const int part = blockIdx.z;
    const int Hq = p.num_q_heads, Hkv = p.num_kv_heads, G = p.group;

    const int L = p.context_lens[s];
    const bool bad_len = L < 0 || static_cast<int64_t>(L) >
                                      static_cast<int64_t>(p.max_blocks_per_seq) * kBlockSize;
    if (bad_len || L == 0) {
        // Partitioned mode leaves these rows to the reduce kernel.
        if (p.out != nullptr && part == 0) {
            const float fill = bad_len ? __builtin_nanf("") : 0.0f;
            for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
                const int h = idx / D, d = idx - (idx / D) * D;
                store_out<OUT>(p.out, ((int64_t)s * Hq + kvh * G + h) * D + d, fill);
            }
        }
        return;
    }
    const int nblk = (L + kBlockSize - 1) / kBlockSize;
    const int pb0 = part * p.partition_blocks;
    if (pb0 >= nblk)
        return;
    const int pb1 = min(pb0 + p.partition_blocks, nblk);
    const int tok_end = min(pb1 * kBlockSize, L);
    const int nb = pb1 - pb0;
    const int nbw = nb > wave ? (nb - wave + nw - 1) / nw : 0;   // this wave's blocks

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

    float* p_lds = smem + wave * 256;
    bool poisoned = false;

    auto load_tile = [&](int phys, Tile<KV, D>& t) {
        const char* kb = kbase + (int64_t)phys * blk_stride + koff;
        const char* vb = vbase + (int64_t)phys * blk_stride + voff;
#pragma unroll
        for (int c = 0; c < NQ; ++c)
            t.k[c] = ld16(kb + 64 * c);
#pragma unroll
        for (int c = 0; c < NV; ++c)
            t.v[c] = ld16(vb + TPL * ROW * c);
    };

    auto process = [&](const Tile<KV, D>& t, int blk) {
        // logits[head 4g+j][token r16]
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < NQ; ++c)
            acc = Op::qk(qa[c], t.k[c], acc);
        const int valid = min(kBlockSize, tok_end - blk * kBlockSize);
        const bool tvalid = r16 < valid;
        float pexp[4], alpha[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float x = tvalid ? acc[j] * p.scale_log2 : -INFINITY;
            const float mn = fmaxf(m[j], row_max16(x));
            alpha[j] = __builtin_amdgcn_exp2f(m[j] - mn);
            pexp[j] = __builtin_amdgcn_exp2f(x - mn);
            lsum[j] = lsum[j] * alpha[j] + pexp[j];
            m[j] = mn;
        }
        *reinterpret_cast<f32x4*>(p_lds + r16 * 16 + 4 * g) = f32x4{pexp[0], pexp[1], pexp[2], pexp[3]};
        float al[GMAX];
#pragma unroll
        for (int h = 0; h < GMAX; ++h)
            al[h] = readlane_f(alpha[h & 3], 16 * (h >> 2));
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int h = 0; h < GMAX; ++h)
#pragma unroll
            for (int e = 0; e < EPC; ++e)
                o[h][e] *= al[h];
#pragma unroll
        for (int c = 0; c < NV; ++c) {
            const int tr = vrow + TPL * c;
            float pv[GMAX];
            if constexpr (GMAX >= 4) {
#pragma unroll
                for (int h4 = 0; h4 < GMAX; h4 += 4) {
                    const f32x4 q4 = *reinterpret_cast<const f32x4*>(p_lds + tr * 16 + h4);
                    pv[h4] = q4[0];
                    pv[h4 + 1] = q4[1];
                    pv[h4 + 2] = q4[2];
                    pv[h4 + 3] = q4[3];
                }
            } else {
#pragma unroll
                for (int h = 0; h < GMAX; ++h)
                    pv[h] = p_lds[tr * 16 + h];
            }
            float vf[EPC];
            Op::to_f32(t.v[c], vf);
            if (valid < kBlockSize && tr >= valid) {
                // Tail rows may hold anything (even NaN): drop them, do not scale them by 0.
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
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    const int64_t tbl = (int64_t)s * p.max_blocks_per_seq + pb0 + wave;
    for (int b0 = 0; b0 < nbw && !poisoned; b0 += kWave) {
        const int nbatch = min(kWave, nbw - b0);
        // Resolve this wave's next (up to) 64 block-table entries at once.
        int phys_l = 0;
        if (lane < nbatch)
            phys_l = p.block_tables[tbl + (int64_t)(b0 + lane) * nw];
        const bool bad = lane < nbatch && (phys_l < 0 || static_cast<int64_t>(phys_l) >= p.num_blocks);
        if (__ballot(bad) != 0) {
            poisoned = true;
            break;
        }
        // Two register tiles in ping-pong: block i+1 is in flight while block i is computed.
        const int jb = pb0 + wave + b0 * nw;      // logical index of the batch's first block
        Tile<KV, D> ta, tb;
        load_tile(__builtin_amdgcn_readlane(phys_l, 0), ta);
        int i = 0;
        for (; i + 2 < nbatch; i += 2) {
            load_tile(__builtin_amdgcn_readlane(phys_l, i + 1), tb);
            process(ta, jb + i * nw);
            load_tile(__builtin_amdgcn_readlane(phys_l, i + 2), ta);
            process(tb, jb + (i + 1) * nw);
        }
        if (i + 1 < nbatch) {
            load_tile(__builtin_amdgcn_readlane(phys_l, i + 1), tb);
            process(ta, jb + i * nw);
            process(tb, jb + (i + 1) * nw);
        } else {
            process(ta, jb + i * nw);
        }
    }

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

    constexpr int GP = padded_group<GMAX>();
    float* red_m = smem + nw * 256;
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

    // Merge the waves in a fixed order and write this workgroup's result.
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
        if (p.out != nullptr) {
            store_out<OUT>(p.out, row * D + d, acc / S);
        } else {
            const int64_t pi = row * p.num_partitions + part;
            p.part_out[pi * D + d] = acc / S;
            if (d == 0) {
                p.part_max[pi] = M * kLn2;
                p.part_sum[pi] = S;
            }
        }
    }
}

// Log-sum-exp combination of the partitions of one (sequence, query head).
template <int D, typename OUT>
__global__ __launch_bounds__(kWave) void lse_reduce_kernel(ReduceParams p) {
    constexpr int DPL = D / kWave;   // output elements per lane (1 or 2)
    const int h = blockIdx.x;
    const int s = blockIdx.y;
    const int lane = threadIdx.x;
    const int Hq = p.num_q_heads, NP = p.num_partitions;
    const int L = p.context_lens[s];
    const int64_t orow = ((int64_t)s * Hq + h) * D;
    const bool bad = L < 0 ||
                     static_cast<int64_t>(L) > static_cast<int64_t>(p.max_blocks_per_seq) * kBlockSize ||
                     static_cast<int64_t>(L) > static_cast<int64_t>(NP) * p.partition_size;
    if (bad || L == 0) {
        const float fill = bad ? __builtin_nanf("") : 0.0f;
#pragma unroll
        for (int k = 0; k < DPL; ++k)
            store_out<OUT>(p.out, orow + lane * DPL + k, fill);
        return;
    }
    const int np = (L + p.partition_size - 1) / p.partition_size;
    const int64_t base = ((int64_t)s * Hq + h) * NP;
    float mx = -INFINITY;
    for (int i = lane; i < np; i += kWave)
        mx = fmaxf(mx, p.part_max[base + i]);
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1)
        mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
    float acc[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k)
        acc[k] = 0.0f;
    float wsum = 0.0f;
    for (int i = 0; i < np; ++i) {
        const float w = p.part_sum[base + i] * __builtin_amdgcn_exp2f((p.part_max[base + i] - mx) * kLog2e);
        wsum += w;
        const float* po = p.part_out + (base + i) * D + lane * DPL;
        if constexpr (DPL == 2) {
            const f32x2 v = *reinterpret_cast<const f32x2*>(po);
            acc[0] = fmaf(w, v[0], acc[0]);
            acc[1] = fmaf(w, v[1], acc[1]);
        } else {
            acc[0] = fmaf(w, po[0], acc[0]);
        }
    }
#pragma unroll
    for (int k = 0; k < DPL; ++k)
        store_out<OUT>(p.out, orow + lane * DPL + k, acc[k] / wsum);
}

template <typename KV, int D, int GMAX, typename OUT>
hipError_t launch_decode_t(const DecodeParams& p, int num_seqs, int grid_partitions, int waves,
                           hipStream_t stream) {
    const size_t lds = decode_lds_bytes<GMAX, D>(waves);
    hipLaunchKernelGGL((paged_decode_kernel<KV, D, GMAX, OUT>),
                       dim3(p.num_kv_heads, num_seqs, grid_partitions), dim3(waves * kWave), lds,
                       stream, p);
    return hipGetLastError();
}

template <typename KV, int D, typename OUT>
hipError_t launch_decode_g(const DecodeParams& p, int num_seqs, int grid_partitions, int waves,
                           hipStream_t stream) {
    const int G = p.group;
    if (G <= 1)
        return launch_decode_t<KV, D, 1, OUT>(p, num_seqs, grid_partitions, waves, stream);
    if (G <= 2)
        return launch_decode_t<KV, D, 2, OUT>(p, num_seqs, grid_partitions, waves, stream);
    if (G <= 4)
        return launch_decode_t<KV, D, 4, OUT>(p, num_seqs, grid_partitions, waves, stream);
    if (G <= 8)
        return launch_decode_t<KV, D, 8, OUT>(p, num_seqs, grid_partitions, waves, stream);
    return launch_decode_t<KV, D, 16, OUT>(p, num_seqs, grid_partitions, waves, stream);
}

template <typename KV, int D>
hipError_t launch_decode_o(const DecodeParams& p, int out_bf16, int num_seqs, int grid_partitions,
                           int waves, hipStream_t stream) {
    return out_bf16 ? launch_decode_g<KV, D, BF16>(p, num_seqs, grid_partitions, waves, stream)
                    : launch_decode_g<KV, D, F32>(p, num_seqs, grid_partitions, waves, stream);
}

}  // namespace

size_t decode_lds_bytes_for(int head_size, int group, int waves) {
    const int gmax = group <= 1 ? 1 : group <= 2 ? 2 : group <= 4 ? 4 : group <= 8 ? 8 : 16;
    const int gp = (gmax + 3) & ~3;
    return sizeof(float) * static_cast<size_t>(waves) * (256 + 2 * gp + gmax * head_size);
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

hipError_t launch_reduce(const ReduceParams& p, int head_size, int out_bf16, int num_seqs,
                         hipStream_t stream) {
    const dim3 grid(p.num_q_heads, num_seqs);
    if (head_size == 64) {
        if (out_bf16)
            hipLaunchKernelGGL((lse_reduce_kernel<64, BF16>), grid, dim3(kWave), 0, stream, p);
        else
            hipLaunchKernelGGL((lse_reduce_kernel<64, F32>), grid, dim3(kWave), 0, stream, p);
    } else {
        if (out_bf16)
            hipLaunchKernelGGL((lse_reduce_kernel<128, BF16>), grid, dim3(kWave), 0, stream, p);
        else
            hipLaunchKernelGGL((lse_reduce_kernel<128, F32>), grid, dim3(kWave), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace pa

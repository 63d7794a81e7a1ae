// pa_device.h -- device helpers shared by the MFMA attention kernels over
// dense query tiles (shared-prefix and multi-token-query kernels).
#pragma once

#include "pa_internal.h"

namespace pa {
namespace dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr float kLn2 = 0.6931471805599453f;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Max / sum over the 16 lanes of a DPP row (quad swaps, then half-row and
// row mirrors); every lane of the row gets the result.
__device__ __forceinline__ float row_max16(float x) {
    x = fmaxf(x, dpp<0xB1>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    x = fmaxf(x, dpp<0x141>(x));
    x = fmaxf(x, dpp<0x140>(x));
    return x;
}

__device__ __forceinline__ float row_sum16(float x) {
    x = x + dpp<0xB1>(x);
    x = x + dpp<0x4E>(x);
    x = x + dpp<0x141>(x);
    x = x + dpp<0x140>(x);
    return x;
}

// Max / sum over the 64 lanes of a wave, returned to every lane: the 16-lane
// row reductions above, then gfx950's row swaps (v_permlane16_swap pairs lane
// l with l ^ 16, v_permlane32_swap with l ^ 32; called with the same value as
// both operands, each lane gets its own value and its partner's), all in the
// VALU. A fixed order: the same inputs always give the same bits.
__device__ __forceinline__ float wave_max(float x) {
    x = row_max16(x);
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t w = __float_as_uint(x);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float wave_sum(float x) {
    x = row_sum16(x);
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t w = __float_as_uint(x);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Inclusive prefix sum over the 64 lanes of a wave (lane i gets x_0 + ... +
// x_i): shifts by 1, 2, 4 and 8 lanes within each 16-lane row (a lane with no
// source adds 0), then lane 15 of rows 0 and 2 added into rows 1 and 3
// (row_bcast:15) and lane 31 into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ int wave_inclusive_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);
    return x;
}

// fp32 -> bf16 bits, round to nearest even (for finite values).
__device__ __forceinline__ uint16_t bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float bf16_value(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even, NaN kept NaN (output rows).
__device__ __forceinline__ uint16_t bf16_out(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return static_cast<uint16_t>((u >> 16) | 0x40u);
    return bf16_bits(x);
}

// Splits eight finite fp32 values into a bf16 high part and the bf16 rounding
// of the remainder (value - high), both round-to-nearest-even, with the
// hardware's packed conversion: together they keep about 16 bits.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split_bf16x8(const float (&v)[8], u16x8& hi, u16x8& lo) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
        const bf16x2 h = {static_cast<__bf16>(v[i]), static_cast<__bf16>(v[i + 1])};
        const uint32_t hb = __builtin_bit_cast(uint32_t, h);
        const float h0 = __uint_as_float(hb << 16), h1 = __uint_as_float(hb & 0xFFFF0000u);
        const bf16x2 l = {static_cast<__bf16>(v[i] - h0), static_cast<__bf16>(v[i + 1] - h1)};
        const uint32_t lb = __builtin_bit_cast(uint32_t, l);
        hi[i] = static_cast<uint16_t>(hb);
        hi[i + 1] = static_cast<uint16_t>(hb >> 16);
        lo[i] = static_cast<uint16_t>(lb);
        lo[i + 1] = static_cast<uint16_t>(lb >> 16);
    }
}

// Workgroup barrier that orders LDS traffic only: global loads in flight stay
// in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroups are dealt to the GPU's 8 XCDs round-robin by their flattened id
// (x fastest). For a grid of n workgroups made of groups of `group` logical
// neighbours (tiles that read the same K/V), this maps flattened id `id` to
// a logical id such that every group runs on one XCD, whose L2 then serves
// its shared reads, and consecutive groups go to different XCDs (so the work
// stays spread over all of them). It is a bijection of [0, n) when the group
// count is a multiple of 8; otherwise the identity is returned. Results never
// depend on it.
__device__ __forceinline__ int64_t xcd_grouped(int64_t id, int64_t n, int64_t group) {
    constexpr int64_t kXcds = 8;
    const int64_t groups = n / group;
    if (groups * group != n || groups % kXcds != 0)
        return id;
    const int64_t x = id % kXcds, k = id / kXcds;
    return (x + kXcds * (k / group)) * group + k % group;
}

}  // namespace dev
}  // namespace pa

// Internal helpers shared by the CSA HIP kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace csa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// s_waitcnt immediate: vmcnt(0), the other counters left free
constexpr int kVmcntZero = 0x0f70;

// float32 -> bfloat16 bits, round to nearest even (quiet NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Order-preserving 32-bit key of a score: larger score <=> larger key.
// -0.0 is folded onto +0.0 first so equal scores get equal keys.
// Keys <= kKeyNegInf belong to -inf (masked) or NaN and are never selected.
constexpr uint32_t kKeyNegInf = 0x007fffffu;
__device__ __forceinline__ uint32_t score_key(float x) {
    uint32_t u = __float_as_uint(x + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ bool key_valid(uint32_t k, float x) {
    return k > kKeyNegInf && x == x;
}

// ---- lane exchanges inside a wave64 without the LDS crossbar ---------------------
// DPP moves serve partners inside a row of 16 lanes, the permlane swaps of
// gfx950 serve partners across rows and wave halves (ds_bpermute, what
// __shfl_xor compiles to, costs an LDS round trip per step).
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kCtrl, 0xf, 0xf, false));
}
constexpr int kDppQuadXor1 = 0xb1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4e;  // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowRor12 = 0x12c;

// v of lane (lane ^ kMask).
template <int kMask>
__device__ __forceinline__ uint32_t xor_lanes(uint32_t v) {
    static_assert(kMask == 1 || kMask == 2 || kMask == 4 || kMask == 8 || kMask == 16 || kMask == 32,
                  "lane mask");
    if constexpr (kMask == 1) {
        return dpp_mov<kDppQuadXor1>(v);
    } else if constexpr (kMask == 2) {
        return dpp_mov<kDppQuadXor2>(v);
    } else if constexpr (kMask == 4) {
        // rotating a row right by 4 brings lane l - 4, by 12 lane l + 4
        const uint32_t down = dpp_mov<kDppRowRor4>(v);
        const uint32_t up = dpp_mov<kDppRowRor12>(v);
        return (__lane_id() & 4) ? down : up;
    } else if constexpr (kMask == 8) {
        return dpp_mov<kDppRowRor8>(v);
    } else if constexpr (kMask == 16) {
        // with both operands v: [0] holds rows 0,0,2,2 and [1] rows 1,1,3,3
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (__lane_id() & 16) ? r[0] : r[1];
    } else {
        // [0] holds the low half twice, [1] the high half twice
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (__lane_id() & 32) ? r[0] : r[1];
    }
}
template <int kMask>
__device__ __forceinline__ float xor_lanes_f32(float v) {
    return __uint_as_float(xor_lanes<kMask>(__float_as_uint(v)));
}
template <int kMask>
__device__ __forceinline__ unsigned long long xor_lanes_u64(unsigned long long v) {
    const uint32_t lo = xor_lanes<kMask>(static_cast<uint32_t>(v));
    const uint32_t hi = xor_lanes<kMask>(static_cast<uint32_t>(v >> 32));
    return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// v of lane (lane ^ o) for o in {1, 2, 4, 8} (unrolled loops give a constant o).
__device__ __forceinline__ float row16_xor(float v, int o) {
    switch (o) {
        case 1: return xor_lanes_f32<1>(v);
        case 2: return xor_lanes_f32<2>(v);
        case 4: return xor_lanes_f32<4>(v);
        default: return xor_lanes_f32<8>(v);
    }
}

// All-lane reductions over the wave (every lane active): rotations inside
// rows of 16 (DPP, fused into the operation by the compiler), then the row
// and half swaps, whose two results together cover both partners.
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce32(T v, Op op) {
    static_assert(sizeof(T) == 4, "32-bit values");
    auto mov = [](T x, auto ctrl) -> T {
        return __builtin_bit_cast(T, dpp_mov<decltype(ctrl)::value>(__builtin_bit_cast(uint32_t, x)));
    };
    v = op(v, mov(v, std::integral_constant<int, kDppQuadXor1>{}));
    v = op(v, mov(v, std::integral_constant<int, kDppQuadXor2>{}));
    v = op(v, mov(v, std::integral_constant<int, kDppRowRor4>{}));
    v = op(v, mov(v, std::integral_constant<int, kDppRowRor8>{}));
    // (vector elements are copied to scalars before any bit cast: a bit cast
    // of an element of the returned pair reads element 0 for both)
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    v = op(__builtin_bit_cast(T, r0), __builtin_bit_cast(T, r1));
    const uint32_t w = __builtin_bit_cast(uint32_t, v);
    const auto q = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    const uint32_t q0 = q[0], q1 = q[1];
    return op(__builtin_bit_cast(T, q0), __builtin_bit_cast(T, q1));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    return wave_reduce32(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
    return wave_reduce32(v, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ float wave_max(float v) {
    return wave_reduce32(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_sum(float v) {
    return wave_reduce32(v, [](float a, float b) { return a + b; });
}
// 64-bit max: the high words first; the low words only decide among the
// lanes that share the top high word (read directly when only one does).
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
    const uint32_t hi = static_cast<uint32_t>(v >> 32);
    const uint32_t lo = static_cast<uint32_t>(v);
    const uint32_t mh = wave_max_u32(hi);
    const unsigned long long tie = __ballot(hi == mh);
    uint32_t ml;
    if (__popcll(tie) == 1)
        ml = static_cast<uint32_t>(
            __builtin_amdgcn_readlane(static_cast<int>(lo), static_cast<int>(__ffsll(static_cast<long long>(tie)) - 1)));
    else
        ml = wave_max_u32(hi == mh ? lo : 0u);
    return (static_cast<unsigned long long>(mh) << 32) | ml;
}

}  // namespace csa

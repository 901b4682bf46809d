// OCP FP8 E4M3 codes (bias 7, subnormals, NaN at S.1111.111, +-448 largest):
// the encoder of the per-row quantiser and an exact decoder, shared by the
// FP8 scan and the decode step's key compressor.
#pragma once

#include "common.h"

namespace csa {

namespace {

// Round to nearest, ties to the even code, saturating at +-448 (integer
// arithmetic on the binary32 bits, no conversion instruction).
__device__ inline uint8_t e4m3_encode_rne(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a >= 0x43e00000u) return static_cast<uint8_t>(sign | 0x7eu);  // |y| >= 448: saturate
    const int e = static_cast<int>(a >> 23) - 127;
    if (e >= -6) {  // normal E4M3
        const uint32_t mant = a & 0x7fffffu;
        uint32_t m3 = mant >> 20;
        const uint32_t rem = mant & 0xfffffu;
        if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ++m3;
        uint32_t ee = static_cast<uint32_t>(e + 7);
        if (m3 == 8u) {
            m3 = 0;
            ++ee;
        }
        return static_cast<uint8_t>(sign | (ee << 3) | m3);
    }
    // subnormal E4M3: m * 2^-9, m = round(|y| * 2^9) in 0..8
    const int sh = 14 - e;  // |y| * 2^9 = (1.mant * 2^23) >> sh
    if (sh >= 25) return static_cast<uint8_t>(sign);  // below half the smallest subnormal
    const uint32_t M = (a & 0x7fffffu) | 0x800000u;
    uint32_t m = M >> sh;
    const uint32_t rem = M & ((1u << sh) - 1u);
    const uint32_t half = 1u << (sh - 1);
    if (rem > half || (rem == half && (m & 1u))) ++m;
    return static_cast<uint8_t>(sign | m);
}

// A row's E4M3 scale (s = amax / 448, 1 for an all-zero row) and what the
// fast quotient below needs: y = 1 / s (both binary32, correctly rounded).
struct E4m3Row {
    float s, y;
    bool recip;  // the reciprocal form is exact for this row
};
__device__ inline E4m3Row e4m3_row(float amax) {
    E4m3Row r;
    r.s = amax > 0.f ? amax / 448.0f : 1.0f;
    r.y = 1.0f / r.s;
    r.recip = amax >= 0x1p-90f || amax == 0.f;
    return r;
}
// RN(x / s) for a bfloat16 value x of the row (|x| <= amax): q = RN(x y),
// then one correction with the exact residual x - s q (Markstein's theorem
// for a correctly rounded reciprocal).  It equals the binary32 division for
// every pair of bfloat16 x and bfloat16 amax >= 2^-90 (an exhaustive host
// check of all 1.06e9 pairs); smaller rows take the division, where the
// residual could underflow.  The quotient has x's sign (also for -0).
__device__ inline float e4m3_quot(float x, const E4m3Row& r) {
    if (!r.recip) return x / r.s;
    float q = x * r.y;
    const float res = __builtin_fmaf(-r.s, q, x);
    q = __builtin_fmaf(res, r.y, q);
    return __builtin_copysignf(q, x);
}
// Codes of two quotients by the conversion instruction (round to nearest
// even): equal to e4m3_encode_rne for every binary32 value of magnitude up
// to 448.0001 (all 2.28e9 of them compared on gfx950), which covers every
// x / s of a row (at most 448 / (1 - 2^-24)).  The low byte is a's code,
// the next b's.
__device__ inline uint32_t e4m3_encode2(float a, float b) {
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xffffu;
}

// The exact value of an E4M3 code (never NaN here: the encoder saturates).
__device__ inline float e4m3_decode(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u;
    const uint32_t m = c & 7u;
    const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : static_cast<float>(m) * 0.001953125f;
    return (c & 0x80u) ? -mag : mag;
}

}  // namespace

}  // namespace csa

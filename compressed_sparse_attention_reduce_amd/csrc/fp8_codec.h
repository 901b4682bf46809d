// OCP FP8 E4M3 codes (bias 7, subnormals, NaN at S.1111.111, +-448 largest):
// the encoder of the per-row quantiser and an exact decoder, shared by the
// FP8 scan and the decode step's key compressor.  Also FP4 E2M1 elements
// with E8M0 block scales (the OCP microscaling element and scale formats:
// magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; a scale is 2^(s - 127)), which
// gfx950's scaled matrix instructions read.
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

// E8M0 exponent X of a 32-element block whose largest magnitude is amax
// (finite, >= 0): the smallest X with amax <= 6 * 2^X, clamped to [-127,
// 127]; 0 for an all-zero block.  With amax = 1.f * 2^E (normal binary32),
// 6 * 2^X = 1.5 * 2^(X + 2), so X = E - 2 when 1.f <= 1.5, else E - 1; a
// subnormal amax (below 2^-126 <= 6 * 2^-127) takes the clamp.
__device__ inline int mx_block_exp(float amax) {
    if (!(amax > 0.f)) return 0;
    const uint32_t u = __float_as_uint(amax);
    const int e = static_cast<int>((u >> 23) & 0xffu);
    if (e == 0) return -127;
    const int x = e - 127 - 2 + ((u & 0x7fffffu) > 0x400000u ? 1 : 0);
    return x < -127 ? -127 : x;
}

// E2M1 code of y (|y| <= 6 after the block scale): round to nearest, ties
// to the even code, saturating at 6; a zero result is code 0 whatever y's
// sign.  The thresholds are the midpoints between neighbouring magnitudes,
// strict where the lower neighbour's code is even.
__device__ inline uint32_t e2m1_encode_rne(float y) {
    const float a = fabsf(y);
    const uint32_t c = static_cast<uint32_t>(a > 0.25f) + static_cast<uint32_t>(a >= 0.75f) +
                       static_cast<uint32_t>(a > 1.25f) + static_cast<uint32_t>(a >= 1.75f) +
                       static_cast<uint32_t>(a > 2.5f) + static_cast<uint32_t>(a >= 3.5f) +
                       static_cast<uint32_t>(a > 5.0f);
    return (y < 0.f && c != 0u) ? (c | 8u) : c;
}

// The exact value of an E2M1 code (low 4 bits of c).
__device__ inline float e2m1_decode(uint32_t c) {
    const uint32_t e = (c >> 1) & 3u;
    const uint32_t m = c & 1u;
    const float mag = e ? __uint_as_float(((e + 126u) << 23) | (m << 22)) : 0.5f * static_cast<float>(m);
    return (c & 8u) ? -mag : mag;
}

}  // namespace

}  // namespace csa

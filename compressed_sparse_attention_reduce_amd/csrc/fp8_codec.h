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

// The exact value of an E4M3 code (never NaN here: the encoder saturates).
__device__ inline float e4m3_decode(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u;
    const uint32_t m = c & 7u;
    const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : static_cast<float>(m) * 0.001953125f;
    return (c & 0x80u) ? -mag : mag;
}

}  // namespace

}  // namespace csa

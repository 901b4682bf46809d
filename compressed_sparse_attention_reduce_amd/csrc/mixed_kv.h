// Mixed main-KV rows: the NoPE part in E4M3 with one row scale, the RoPE
// part in bfloat16 — page 2, single_shot_inference.py, eager_attention (the
// "B1 storage-native mixed path": kv_quantize's E4M3 NoPE codes and scale,
// the RoPE part kept in bfloat16 and rotated at the entry's position;
// "Inverse RoPE" on the attention output).  The pairing of the RoPE dims is
// that of page 1, PERFORMANCE_AUDIT.md P5 (_apply_rope: even / odd entries
// of the trailing rope_dim).
//
// One row is one 592-byte record (d = 512, 64 RoPE dims), 16-byte aligned:
//   bytes   0 .. 447  E4M3 codes of the NoPE part (OCP E4M3, as csa_quantize_fp8)
//   bytes 448 .. 575  the 64 RoPE values, bfloat16
//   bytes 576 .. 579  float32 scale of the codes (max |NoPE| / 448, 1 for zero)
//   bytes 580 .. 591  zero
#pragma once

#include "common.h"
#include "fp8_codec.h"
#include "kernels.h"

namespace csa {

namespace {

// Rotate the RoPE pair (e, o) by the table entry (c, s): forward
// (e c - o s, e s + o c), inverse (e c + o s, -e s + o c).
__device__ __forceinline__ void rope_pair(float& e, float& o, float c, float s, bool inverse) {
    const float e0 = e, o0 = o;
    if (inverse) {
        e = e0 * c + o0 * s;
        o = -e0 * s + o0 * c;
    } else {
        e = e0 * c - o0 * s;
        o = e0 * s + o0 * c;
    }
}

__device__ __forceinline__ float bf16_round(float x) { return bf16_to_f32(f32_to_bf16(x)); }

// One wave writes the record of a row whose value j is get(j) (float32):
// the NoPE part quantised as csa_quantize_fp8 does (binary32 division by the
// scale, nearest-even codes), the RoPE part rounded to bfloat16 and, with a
// table row (cos, sin: kMixRope / 2 values), rotated and rounded again.
template <class Get>
__device__ inline void wave_pack_mixed(Get get, uint8_t* rec, const float* cos, const float* sin) {
    const int lane = threadIdx.x & (kWave - 1);
    constexpr int kPer = kMixNope / kWave;  // 7 NoPE values per lane, consecutive
    static_assert(kPer * kWave == kMixNope, "whole NoPE values per lane");
    float v[kPer];
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        v[e] = get(kPer * lane + e);
        amax = fmaxf(amax, fabsf(v[e]));
    }
    amax = wave_max(amax);
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
    for (int e = 0; e < kPer; ++e) rec[kPer * lane + e] = e4m3_encode_rne(v[e] / scale);
    if (lane < kMixRope / 2) {
        float ev = bf16_round(get(kMixNope + 2 * lane));
        float od = bf16_round(get(kMixNope + 2 * lane + 1));
        if (cos) rope_pair(ev, od, cos[lane], sin[lane], false);
        const uint32_t packed = static_cast<uint32_t>(f32_to_bf16(ev)) | (static_cast<uint32_t>(f32_to_bf16(od)) << 16);
        *reinterpret_cast<uint32_t*>(rec + kMixNope + 4 * lane) = packed;
    } else if (lane == kMixRope / 2) {
        *reinterpret_cast<float*>(rec + kMixScaleOff) = scale;
    } else if (lane < kMixRope / 2 + 4) {
        *reinterpret_cast<uint32_t*>(rec + kMixScaleOff + 4 * (lane - kMixRope / 2)) = 0u;
    }
}

// Eight E4M3 codes (two words) times the row scale, as eight bfloat16
// (nearest even) in a 16-byte piece: v_cvt_pk_f32_fp8 decodes two codes
// exactly (gfx950 reads OCP E4M3), one float32 multiply each, and
// v_cvt_pk_bf16_f32 rounds a pair.
__device__ __forceinline__ uint4 decode8_bf16(uint32_t lo, uint32_t hi, float scale) {
    auto pack = [scale](decltype(__builtin_amdgcn_cvt_pk_f32_fp8(0, false)) f) -> uint32_t {
        const __bf16 a = static_cast<__bf16>(f[0] * scale);
        const __bf16 b = static_cast<__bf16>(f[1] * scale);
        return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
               (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
    };
    return make_uint4(pack(__builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(lo), false)),
                      pack(__builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(lo), true)),
                      pack(__builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(hi), false)),
                      pack(__builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(hi), true)));
}

// Loaders read a 16-byte output piece cc of a record in two steps, so that
// every piece's loads are issued before any of them is used (a load whose
// result is chosen between branches makes the compiler wait for it at the
// join): mixed_piece_ptr gives the bytes to read without branching on the
// piece kind (piece cc < kMixNope / 8: its 8 codes, read as the 16 bytes at
// 8 * cc, which the record holds; otherwise 16 bytes of the RoPE part), and
// after the loads mixed_piece_value turns them and the row scale into 8
// bfloat16 values.
__device__ __forceinline__ const uint8_t* mixed_piece_ptr(const uint8_t* rec, int cc) {
    const bool code = cc < kMixNope / 8;
    return rec + (code ? 8 * cc : kMixNope + 16 * (cc - kMixNope / 8));
}
__device__ __forceinline__ uint4 mixed_piece_load(const uint8_t* p) {  // p: 8-byte aligned
    uint4 v;
    __builtin_memcpy(&v, __builtin_assume_aligned(p, 8), sizeof(v));
    return v;
}

__device__ __forceinline__ uint4 mixed_piece_value(const uint4& raw, float scale, int cc) {
    return cc < kMixNope / 8 ? decode8_bf16(raw.x, raw.y, scale) : raw;
}

}  // namespace

}  // namespace csa

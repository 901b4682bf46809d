// The small per-sequence jobs of a decode step, one workgroup each:
//   role 0  append the new token's KV row to the SWA ring (page 1, P2: the
//           token lands in slot swa_head);
//   role 1  compress the block the token completes into comp_kv[n_comp];
//   role 2  compress that block's indexer key into idx_keys[n_comp] (none
//           for a layer without an indexer: idx_keys == nullptr).
// Roles 1 and 2 run only when the token completes a block.  A long main
// block (main_wgs > 1: HCA ratios, no norm) is split over roles
// 1 .. main_wgs by channel ranges instead, with no indexer role.
#pragma once

#include "compress_impl.h"
#include "fp8_codec.h"
#include "kernels.h"
#include "mixed_kv.h"

namespace csa {

// ybuf: kPrepMaxD floats of LDS; red: blockDim/64 floats of LDS.  key (LDS,
// may be ybuf): role 2 leaves the stored key there as floats (synchronised);
// with E4M3 keys (idx_fp8) key must be d_i + 1 floats apart from ybuf, and
// holds the decoded codes then the row scale.  prev_main / prev_idx: where
// the previous block's rows sit relative to the block's first row (0: just
// before it).
__device__ inline void step_prep_role_at(const PrepArgs& a, int role, int b, float* ybuf, float* red, float* key,
                                         long long prev_main, long long prev_idx) {
    if (role == 0 && a.kv_mixed) {  // the new (rotated) row packed into its ring slot by one wave
        if (threadIdx.x < kWave) {
            const uint16_t* src = static_cast<const uint16_t*>(a.kv_new) + b * a.kv_new_stride_b;
            uint8_t* rec = static_cast<uint8_t*>(a.swa) + b * a.swa_stride_b + static_cast<long long>(a.swa_slot) * kMixRec;
            wave_pack_mixed([&](int j) { return bf16_to_f32(src[j]); }, rec, nullptr, nullptr);
        }
        return;
    }
    if (role == 0) {
        const char* src = static_cast<const char*>(a.kv_new) + b * a.kv_new_stride_b * a.es;
        char* dst = static_cast<char*>(a.swa) + (b * a.swa_stride_b + static_cast<long long>(a.swa_slot) * a.d) * a.es;
        for (int o = threadIdx.x * 16; o < a.d * a.es; o += blockDim.x * 16)
            *reinterpret_cast<uint4*>(dst + o) = *reinterpret_cast<const uint4*>(src + o);
        return;
    }
    if (!a.completes) return;
    if (a.main_wgs > 1) {  // roles 1 .. main_wgs: channel slices of a long main block
        if (role > a.main_wgs) return;
        const int nch = (a.d + a.main_wgs - 1) / a.main_wgs;
        const float* z = a.z_main + b * a.zc_main_stride_b;
        const float* c = a.c_main + b * a.zc_main_stride_b;
        char* out = static_cast<char*>(a.comp_kv) +
                    (b * a.comp_kv_stride_b + static_cast<long long>(a.n_comp) * a.d) * a.es;
        compress_block_slice(z, c, a.main_bias, out, a.es == 2, a.m, a.d, (role - 1) * nch, nch, ybuf);
        return;
    }
    const bool main = role == 1;
    if (main && a.kv_mixed) {
        // the entry in float32 (LDS past the compressor's own buffer), then
        // one wave packs it with its RoPE dims rotated at the block index
        float* y = ybuf + kPrepMaxD / 2;
        const float* z = a.z_main + b * a.zc_main_stride_b;
        const float* c = a.c_main + b * a.zc_main_stride_b;
        compress_block(z, c, a.main_bias, a.main_norm, y, false, a.m, a.d, a.overlap != 0, a.block, ybuf, red,
                       nullptr, prev_main);
        __syncthreads();
        if (threadIdx.x < kWave) {
            uint8_t* rec = static_cast<uint8_t*>(a.comp_kv) + b * a.comp_kv_stride_b +
                           static_cast<long long>(a.n_comp) * kMixRec;
            wave_pack_mixed([&](int j) { return y[j]; }, rec, a.entry_cos, a.entry_sin);
        }
        return;
    }
    if (!main && !a.idx_keys) return;  // a layer without an indexer (HCA)
    if (!main && a.idx_fp8) {
        // E4M3 indexer keys: the key in float32 (in `key`), quantised like
        // csa_quantize_fp8 (scale = max|y| / 448, 1 for a zero row, codes by
        // round to nearest even of y / scale); `key` is left holding the
        // decoded codes and key[a.d_i] the scale (synchronised)
        const float* z = a.z_idx + b * a.zc_idx_stride_b;
        const float* c = a.c_idx + b * a.zc_idx_stride_b;
        compress_block(z, c, a.idx_bias, a.idx_norm, key, false, a.m, a.d_i, a.overlap != 0, a.block, ybuf, red,
                       nullptr, prev_idx);
        __syncthreads();
        if (a.idx_fp4) {
            // FP4 keys (d_i = 128): quantised like csa_quantize_fp4 by the
            // first wave, lane l taking elements 2 l, 2 l + 1 (a 32-element
            // block is 16 lanes); `key` is left holding the decoded values
            // (code times block scale) and key[a.d_i] = 1
            if (a.idx_keys_exact) {  // the key in bfloat16 too (the bfloat16 step's rounding)
                uint16_t* ex = a.idx_keys_exact + b * a.idx_keys_exact_stride_b + static_cast<long long>(a.n_comp) * a.d_i;
                for (int j = threadIdx.x; j < a.d_i; j += blockDim.x) ex[j] = f32_to_bf16(key[j]);
            }
            __syncthreads();  // every thread has read key before the first wave rewrites it
            if (threadIdx.x < kWave) {
                const int l = threadIdx.x;
                const float x0 = key[2 * l], x1 = key[2 * l + 1];
                float amax = fmaxf(fabsf(x0), fabsf(x1));
                amax = fmaxf(amax, xor_lanes_f32<1>(amax));
                amax = fmaxf(amax, xor_lanes_f32<2>(amax));
                amax = fmaxf(amax, xor_lanes_f32<4>(amax));
                amax = fmaxf(amax, xor_lanes_f32<8>(amax));
                const int xe = mx_block_exp(amax);
                const uint32_t c0 = e2m1_encode_rne(__builtin_ldexpf(x0, -xe));
                const uint32_t c1 = e2m1_encode_rne(__builtin_ldexpf(x1, -xe));
                uint8_t* codes = static_cast<uint8_t*>(a.idx_keys) + b * a.idx_keys_stride_b +
                                 static_cast<long long>(a.n_comp) * (a.d_i / 2);
                codes[l] = static_cast<uint8_t>(c0 | (c1 << 4));
                if ((l & 15) == 0)
                    reinterpret_cast<uint8_t*>(a.idx_scales + b * a.idx_scales_stride_b + a.n_comp)[l >> 4] =
                        static_cast<uint8_t>(xe + 127);
                key[2 * l] = __builtin_ldexpf(e2m1_decode(c0), xe);
                key[2 * l + 1] = __builtin_ldexpf(e2m1_decode(c1), xe);
                if (l == 0) key[a.d_i] = 1.0f;
            }
            __syncthreads();
            return;
        }
        float amax = 0.f;
        for (int j = threadIdx.x; j < a.d_i; j += blockDim.x) amax = fmaxf(amax, fabsf(key[j]));
        amax = wave_max(amax);
        if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = amax;
        __syncthreads();
        amax = 0.f;
        for (int w = 0; w < static_cast<int>(blockDim.x / kWave); ++w) amax = fmaxf(amax, red[w]);
        const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
        uint8_t* codes = static_cast<uint8_t*>(a.idx_keys) + b * a.idx_keys_stride_b +
                         static_cast<long long>(a.n_comp) * a.d_i;
        if (a.idx_keys_exact) {  // the key in bfloat16 too (the bfloat16 step's rounding)
            uint16_t* ex = a.idx_keys_exact + b * a.idx_keys_exact_stride_b + static_cast<long long>(a.n_comp) * a.d_i;
            for (int j = threadIdx.x; j < a.d_i; j += blockDim.x) ex[j] = f32_to_bf16(key[j]);
        }
        __syncthreads();  // every thread has read red
        for (int j = threadIdx.x; j < a.d_i; j += blockDim.x) {
            const uint8_t q = e4m3_encode_rne(key[j] / scale);
            codes[j] = q;
            key[j] = e4m3_decode(q);
        }
        if (threadIdx.x == 0) {
            a.idx_scales[b * a.idx_scales_stride_b + a.n_comp] = scale;
            key[a.d_i] = scale;
        }
        __syncthreads();
        return;
    }
    const int d = main ? a.d : a.d_i;
    const float* z = (main ? a.z_main : a.z_idx) + b * (main ? a.zc_main_stride_b : a.zc_idx_stride_b);
    const float* c = (main ? a.c_main : a.c_idx) + b * (main ? a.zc_main_stride_b : a.zc_idx_stride_b);
    char* out = static_cast<char*>(main ? a.comp_kv : a.idx_keys) +
                (b * (main ? a.comp_kv_stride_b : a.idx_keys_stride_b) + static_cast<long long>(a.n_comp) * d) * a.es;
    compress_block(z, c, main ? a.main_bias : a.idx_bias, main ? a.main_norm : a.idx_norm, out, a.es == 2, a.m, d,
                   a.overlap != 0, a.block, ybuf, red, main ? nullptr : key, main ? prev_main : prev_idx);
}

// The jobs with the counters on the device (a.dev): this step's completion,
// entry index, block and ring slot come from *a.dev; the block's Z/C rows
// from a ring of two blocks per array that every step adds its token's rows
// to (role 0 when no block completes; roles 1 and 2 their own arrays, just
// before compressing from the ring, when one does).
__device__ inline void step_prep_role(const PrepArgs& a, int role, int b, float* ybuf, float* red,
                                      float* key = nullptr) {
    if (!a.dev) {
        step_prep_role_at(a, role, b, ybuf, red, key, 0, 0);
        return;
    }
    const DevState st = dev_load(a.dev, a.swa_w, a.max_comp);
    PrepArgs p = a;
    p.completes = dev_completes(st, a.m, a.max_comp) ? 1 : 0;
    p.n_comp = st.n_comp;
    p.block = st.pos / a.m;
    p.swa_slot = st.swa_head;
    if (p.kv_mixed && p.completes) {
        const long long row = p.block < a.comp_rope_rows ? p.block : a.comp_rope_rows - 1;
        p.entry_cos = a.comp_rope_cos + row * (kMixRope / 2);
        p.entry_sin = a.comp_rope_sin + row * (kMixRope / 2);
    }
    const int wm = a.overlap ? 2 * a.d : a.d;
    const int wi = a.overlap ? 2 * a.d_i : a.d_i;
    float* ring = a.dev_ring + b * a.ring_stride_b;
    float* rz_main = ring;
    float* rc_main = ring + 2LL * a.m * wm;
    float* rz_idx = ring + 4LL * a.m * wm;
    float* rc_idx = rz_idx + 2LL * a.m * wi;
    const int slot = st.pos % (2 * a.m);
    auto put = [&](float* dst, const float* src, int width) {
        for (int j = threadIdx.x; j < width; j += blockDim.x) dst[static_cast<long long>(slot) * width + j] = src[j];
    };
    const float* nz_main = a.z_main + b * a.zc_main_stride_b;
    const float* nc_main = a.c_main + b * a.zc_main_stride_b;
    const float* nz_idx = a.z_idx + b * a.zc_idx_stride_b;
    const float* nc_idx = a.c_idx + b * a.zc_idx_stride_b;
    const bool idx = a.idx_keys != nullptr;
    if (role == 0 && !p.completes) {
        put(rz_main, nz_main, wm);
        put(rc_main, nc_main, wm);
        if (idx) {
            put(rz_idx, nz_idx, wi);
            put(rc_idx, nc_idx, wi);
        }
    } else if (p.completes && (role == 1 || (role == 2 && idx))) {
        if (role == 1) {
            put(rz_main, nz_main, wm);
            put(rc_main, nc_main, wm);
        } else {
            put(rz_idx, nz_idx, wi);
            put(rc_idx, nc_idx, wi);
        }
        __syncthreads();  // the ring rows of this workgroup's array are complete
    }
    // the block's first row in the ring, and where the previous block's are
    const long long cur = (p.block & 1) * static_cast<long long>(a.m);
    const long long prev_rows = (1 - 2 * (p.block & 1)) * static_cast<long long>(a.m);
    p.z_main = rz_main + cur * wm;
    p.c_main = rc_main + cur * wm;
    p.z_idx = rz_idx + cur * wi;
    p.c_idx = rc_idx + cur * wi;
    p.zc_main_stride_b = 0;  // already this sequence's ring
    p.zc_idx_stride_b = 0;
    step_prep_role_at(p, role, b, ybuf, red, key, prev_rows * wm, prev_rows * wi);
}

}  // namespace csa

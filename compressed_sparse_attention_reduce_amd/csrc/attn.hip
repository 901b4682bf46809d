// Shared-KV sparse attention over gather_buf with a per-head sink logit.
//
// Page 1, fmha_6warp_tma_multirow_multitile.cuh, hunk "Sink bias correction
// (D5c: single softmax over [S_comp, S_swa + sink])": one softmax over all
// gathered rows plus a per-head sink that adds exp(sink - M) to the
// denominator and has no value row; the sink is already in the scaled domain.
// K = V (page 1, PERFORMANCE_AUDIT.md P4; MQA, one KV head for all heads).
//
// bf16 path, split-K ("flash decoding") in two launches:
//   k_attn_partial_bf16 — grid (row split, group of 16 heads, sequence).  The
//     split's rows are loaded once into LDS with 16-byte lanes (zero-filled
//     past n_valid).  In gather mode (the fused decode step) the rows come
//     straight from the compressed cache through the top-k indices and from the
//     SWA ring, and the head-group-0 workgroups also write them to gather_buf,
//     so the gather costs no launch and no second pass.  Each wave computes
//     S = q K^T for 16 rows on v_mfma_f32_16x16x32_bf16 with the query staged
//     in LDS; the split's softmax statistics are combined across waves in LDS;
//     O = P V runs on the same MFMA with V read column-wise from LDS.  Partial
//     (m, l, O) go to the workspace in float32.
//   k_attn_merge — one workgroup per (head, 128 columns, sequence): M = max(max_s m_s, sink),
//     rescale and add the partials, add exp(sink - M) once, divide.
// float32 path (small correctness workloads): one workgroup per (head,
// sequence), the whole softmax in float32 on the vector ALUs.
#include "common.h"
#include "kernels.h"
#include "attn_split.h"

namespace csa {

namespace {

__global__ __launch_bounds__(kAttnThreads) void k_attn_partial_bf16(AttnArgs a, int n_splits) {
    if (a.dev) attn_dev_view(a, blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0);
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    uint4 qv[AttnSplit<kAttnThreads>::kQBatch];
    attn_load_q<kAttnThreads>(a, blockIdx.y, blockIdx.z, qv);
    attn_split<kAttnThreads>(a, n_splits, blockIdx.x, blockIdx.y, blockIdx.z,
                             a.idx ? a.idx + static_cast<long long>(blockIdx.z) * a.k : nullptr, -1, qv, smem);
}

constexpr int kMaxSplits = 256;
constexpr int kMergeWaves = kAttnThreads / kWave;
// One workgroup per (head, C * 64 columns, sequence): C = 2 while the
// workgroups would not fill the chip twice over, else 4 (16-byte loads, half
// the workgroups).  Every wave derives the
// split weights itself (lane s holds split s of each group of 64, no
// barrier); wave w sums splits w, w + 4, ... for the workgroup's columns and
// the four partial sums meet in LDS.  Partials of empty splits (l = 0) are
// never written: their loads read stale workspace bytes that are skipped
// (never multiplied).
template <int C>
__global__ __launch_bounds__(kAttnThreads) void k_attn_merge(const float* __restrict__ ws_o,
                                                             const float* __restrict__ ws_ml,
                                                             const float* __restrict__ sink, int h,
                                                             int d, int n_splits, void* __restrict__ out,
                                                             int out_bf16, float* __restrict__ lse,
                                                             long long out_stride_b, const float* inv_cos,
                                                             const float* inv_sin, int rope_start,
                                                             const int* dev_pos, const float* rope_cos,
                                                             const float* rope_sin, int rope_rows, DevState* adv,
                                                             int adv_m, int adv_w, int adv_max_comp) {
    __shared__ float4 part[kMergeWaves][kWave];
    if (dev_pos && rope_cos) {  // the inverse-RoPE row of the step's position (device counters)
        const int p = *dev_pos < rope_rows ? *dev_pos : rope_rows - 1;
        const long long row = static_cast<long long>(p) * (kMixRope / 2);
        inv_cos = rope_cos + row;
        inv_sin = rope_sin + row;
    }
    static_assert(C == 2 || C == 4, "column pairs or quads per lane");
    constexpr int kCols = C * kWave;
    const int col_blocks = (d + kCols - 1) / kCols;
    const int hh = blockIdx.x / col_blocks;
    const int cb = blockIdx.x % col_blocks;
    const int b = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const long long base = (static_cast<long long>(b) * h + hh) * n_splits;
    const float* ml = ws_ml + 2 * base;
    const float* ob = ws_o + base * d;
    const int col = cb * kCols + C * lane;
    const bool has_col = col < d;  // d is a multiple of 32
    auto load = [&](int sp) -> float4 {
        if (!has_col || sp >= n_splits) return make_float4(0.f, 0.f, 0.f, 0.f);
        const float* p = ob + static_cast<long long>(sp) * d + col;
        if constexpr (C == 4) return *reinterpret_cast<const float4*>(p);
        const float2 t = *reinterpret_cast<const float2*>(p);
        return make_float4(t.x, t.y, 0.f, 0.f);
    };
    // this wave's first splits' loads go first
    constexpr int kBatch = 16;
    float4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) v[u] = load(wv + kMergeWaves * u);
    constexpr int kGroups = kMaxSplits / kWave;
    float ms[kGroups], ls[kGroups];
    float M = sink ? sink[hh] : -INFINITY;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
        const int sp = g * kWave + lane;
        ms[g] = sp < n_splits ? ml[2 * sp] : -INFINITY;
        ls[g] = sp < n_splits ? ml[2 * sp + 1] : 0.f;
        if (ls[g] > 0.f) M = fmaxf(M, ms[g]);
    }
    M = wave_max(M);
    float den = 0.f;
    if (M != -INFINITY)
#pragma unroll
        for (int g = 0; g < kGroups; ++g)
            if (ls[g] > 0.f) den += ls[g] * expf(ms[g] - M);
    den = wave_sum(den);
    if (M != -INFINITY && sink) den += expf(sink[hh] - M);
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    float cf[kGroups];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) cf[g] = (ls[g] > 0.f && M != -INFINITY) ? expf(ms[g] - M) * inv : 0.f;
    auto coef = [&](int sp) -> float {  // sp is uniform: one scalar read of lane sp % 64
        float c = 0.f;
#pragma unroll
        for (int g = 0; g < kGroups; ++g)
            if (sp / kWave == g) c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cf[g]), sp % kWave));
        return c;
    };
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < n_splits; s0 += kMergeWaves * kBatch) {
        if (s0 > 0) {
#pragma unroll
            for (int u = 0; u < kBatch; ++u) v[u] = load(s0 + wv + kMergeWaves * u);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int sp = s0 + wv + kMergeWaves * u;
            if (sp < n_splits) {
                const float c = coef(sp);
                if (c != 0.f) {
                    acc.x += v[u].x * c;
                    acc.y += v[u].y * c;
                    if constexpr (C == 4) {
                        acc.z += v[u].z * c;
                        acc.w += v[u].w * c;
                    }
                }
            }
        }
    }
    part[wv][lane] = acc;
    __syncthreads();
    if (wv != 0) return;
#pragma unroll
    for (int w = 1; w < kMergeWaves; ++w) {
        const float4 o = part[w][lane];
        acc.x += o.x;
        acc.y += o.y;
        acc.z += o.z;
        acc.w += o.w;
    }
    if (has_col) {
        // the RoPE dims rotated back at the token's position (a lane holds
        // two (even, odd) pairs)
        if (inv_cos && col >= rope_start) {
            const int pr = (col - rope_start) / 2;
            rope_pair(acc.x, acc.y, inv_cos[pr], inv_sin[pr], true);
            if constexpr (C == 4) rope_pair(acc.z, acc.w, inv_cos[pr + 1], inv_sin[pr + 1], true);
        }
        const long long o = b * out_stride_b + static_cast<long long>(hh) * d + col;
        const float y[4] = {acc.x, acc.y, acc.z, acc.w};
        if (out_bf16) {
            uint16_t* p = static_cast<uint16_t*>(out) + o;
            if (C == 4 && (reinterpret_cast<uintptr_t>(p) & 7) == 0) {  // one 8-byte store
                *reinterpret_cast<uint2*>(p) =
                    make_uint2(f32_to_bf16(y[0]) | (static_cast<uint32_t>(f32_to_bf16(y[1])) << 16),
                               f32_to_bf16(y[2]) | (static_cast<uint32_t>(f32_to_bf16(y[3])) << 16));
            } else {
#pragma unroll
                for (int e = 0; e < C; ++e) p[e] = f32_to_bf16(y[e]);
            }
        } else {
            float* p = static_cast<float*>(out) + o;
            if (C == 4 && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {  // one 16-byte store
                *reinterpret_cast<float4*>(p) = acc;
            } else {
#pragma unroll
                for (int e = 0; e < C; ++e) p[e] = y[e];
            }
        }
    }
    if (lse && cb == 0 && lane == 0)
        lse[static_cast<long long>(b) * h + hh] = den > 0.f ? M + logf(den) : -INFINITY;
    // device counters: the step's other kernels have read them (stream order)
    // and no workgroup of this one does
    if (adv && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) dev_advance(adv, adv_m, adv_w, adv_max_comp);
}

// float32 path
constexpr int kAttnF32Threads = 256;

__device__ inline float block_reduce_max(float v, float* red) {
    v = wave_max(v);
    const int wv = threadIdx.x / kWave;
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) red[wv] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < static_cast<int>(blockDim.x / kWave); ++i) r = fmaxf(r, red[i]);
    return r;
}
__device__ inline float block_reduce_sum(float v, float* red) {
    v = wave_sum(v);
    const int wv = threadIdx.x / kWave;
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) red[wv] = v;
    __syncthreads();
    float r = 0.f;
    for (int i = 0; i < static_cast<int>(blockDim.x / kWave); ++i) r += red[i];
    return r;
}

__global__ __launch_bounds__(kAttnF32Threads) void k_attn_f32(
    const float* __restrict__ q, const float* __restrict__ kv, const int* __restrict__ n_valid,
    const float* __restrict__ sink, float scale, void* __restrict__ out, int out_bf16,
    float* __restrict__ lse, int h, int d, int n_max, long long q_stride_b, long long kv_stride_b,
    long long out_stride_b) {
    extern __shared__ float sm[];  // [d] query, then [n_max] logits / weights
    __shared__ float red[kAttnF32Threads / kWave];
    float* qs = sm;
    float* ps = sm + d;
    const int hh = blockIdx.x;
    const int b = blockIdx.y;
    int nv = n_valid[b];
    nv = nv < 0 ? 0 : (nv > n_max ? n_max : nv);
    const float* qh = q + b * q_stride_b + static_cast<long long>(hh) * d;
    const float* kvb = kv + b * kv_stride_b;
    for (int i = threadIdx.x; i < d; i += blockDim.x) qs[i] = qh[i];
    __syncthreads();
    float mx = sink ? sink[hh] : -INFINITY;
    for (int j = threadIdx.x; j < nv; j += blockDim.x) {
        const float* r = kvb + static_cast<long long>(j) * d;
        float dot = 0.f;
        for (int i = 0; i < d; ++i) dot += qs[i] * r[i];
        ps[j] = dot * scale;
        mx = fmaxf(mx, ps[j]);
    }
    const float M = block_reduce_max(mx, red);
    float sum = 0.f;
    if (M != -INFINITY) {
        for (int j = threadIdx.x; j < nv; j += blockDim.x) {
            const float p = expf(ps[j] - M);
            ps[j] = p;
            sum += p;
        }
    }
    float den = block_reduce_sum(sum, red);
    if (M != -INFINITY && sink) den += expf(sink[hh] - M);
    __syncthreads();
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    for (int i = threadIdx.x; i < d; i += blockDim.x) {
        float acc = 0.f;
        for (int j = 0; j < nv; ++j) acc += ps[j] * kvb[static_cast<long long>(j) * d + i];
        const float y = acc * inv;
        const long long o = b * out_stride_b + static_cast<long long>(hh) * d + i;
        if (out_bf16) static_cast<uint16_t*>(out)[o] = f32_to_bf16(y);
        else static_cast<float*>(out)[o] = y;
    }
    if (lse && threadIdx.x == 0)
        lse[static_cast<long long>(b) * h + hh] = den > 0.f ? M + logf(den) : -INFINITY;
}

}  // namespace

size_t attn_workspace_bytes(bool bf16, int batch, int h, int d, int n_max) {
    if (!bf16) return 0;
    const size_t ns = static_cast<size_t>(attn_splits(n_max));
    return sizeof(float) * static_cast<size_t>(batch) * h * ns * (static_cast<size_t>(d) + 2);
}

int attn_max_splits() { return kMaxSplits; }

int attn_max_rows() { return kMaxSplits * 32; }

hipError_t launch_attn_bf16(AttnArgs a, hipStream_t s) {
    const int ns = attn_splits(a.n_max);
    a.ws_o = static_cast<float*>(a.ws);
    a.ws_ml = a.ws_o + static_cast<size_t>(a.batch) * a.h * ns * a.d;
    const size_t lds = attn_split_lds_bytes(a.d);
    hipLaunchKernelGGL(k_attn_partial_bf16, dim3(ns, a.h / kHeadGroup, a.batch), dim3(kAttnThreads), lds, s, a, ns);
    return launch_attn_merge(a, ns, s);
}

hipError_t launch_attn_merge(const AttnArgs& a, int ns, hipStream_t s) {
    const bool quads = static_cast<long long>(a.h) * ((a.d + 2 * kWave - 1) / (2 * kWave)) * a.batch >
                       2LL * device_cu_count();
    const int cols = (quads ? 4 : 2) * kWave;
    const dim3 grid(a.h * ((a.d + cols - 1) / cols), a.batch);
    if (quads)
        hipLaunchKernelGGL(k_attn_merge<4>, grid, dim3(kAttnThreads), 0, s, a.ws_o, a.ws_ml, a.sink, a.h, a.d, ns,
                           a.out, a.out_bf16 ? 1 : 0, a.lse, a.out_stride_b, a.inv_cos, a.inv_sin, a.d - kMixRope,
                           a.dev_pos, a.kv_mixed ? a.rope_cos : nullptr, a.rope_sin, a.rope_rows, a.dev_adv, a.m,
                           a.w, a.max_comp);
    else
        hipLaunchKernelGGL(k_attn_merge<2>, grid, dim3(kAttnThreads), 0, s, a.ws_o, a.ws_ml, a.sink, a.h, a.d, ns,
                           a.out, a.out_bf16 ? 1 : 0, a.lse, a.out_stride_b, a.inv_cos, a.inv_sin, a.d - kMixRope,
                           a.dev_pos, a.kv_mixed ? a.rope_cos : nullptr, a.rope_sin, a.rope_rows, a.dev_adv, a.m,
                           a.w, a.max_comp);
    return hipGetLastError();
}

hipError_t launch_attn_f32(const void* q, const void* kv, const int* n_valid, const float* sink,
                           float scale, void* out, bool out_bf16, float* lse, int batch, int h,
                           int d, int n_max, long long q_stride_b, long long kv_stride_b,
                           long long out_stride_b, hipStream_t s) {
    const size_t lds = sizeof(float) * (static_cast<size_t>(d) + (n_max > 0 ? n_max : 1));
    hipLaunchKernelGGL(k_attn_f32, dim3(h, batch), dim3(kAttnF32Threads), lds, s,
                       static_cast<const float*>(q), static_cast<const float*>(kv), n_valid, sink,
                       scale, out, out_bf16 ? 1 : 0, lse, h, d, n_max, q_stride_b, kv_stride_b,
                       out_stride_b);
    return hipGetLastError();
}

}  // namespace csa

// Shared-KV sparse attention over gather_buf with a per-head sink logit.
//
// Page 1, fmha_6warp_tma_multirow_multitile.cuh, hunk "Sink bias correction
// (D5c: single softmax over [S_comp, S_swa + sink])": one softmax over all
// gathered rows plus a per-head sink that adds exp(sink - M) to the
// denominator and has no value row; the sink is already in the scaled domain.
// K = V (page 1, PERFORMANCE_AUDIT.md P4; MQA, one KV head for all heads).
//
// bf16 path, split-K ("flash decoding") in two launches:
//   k_attn_partial_bf16 — grid (row split of 32, group of 16 heads, sequence).
//     The 32 x d key/value tile is loaded once into LDS (coalesced 16 B
//     lanes; rows past n_valid are zero-filled).  S = q K^T on
//     v_mfma_f32_16x16x32_bf16 with the d contraction split over the 4 waves,
//     a local softmax (max m, sum l of the bf16-rounded weights), then
//     O = P V on the same MFMA with V read from LDS column-wise.  Partial
//     (m, l, O) go to the workspace in float32.
//   k_attn_merge — per (head, sequence): M = max(max m_s, sink), rescale and
//     add the partials, add exp(sink - M) to the denominator once, divide.
// float32 path (small correctness workloads): one workgroup per (head,
// sequence) computing the whole softmax in float32 on the vector ALUs.
#include "common.h"
#include "kernels.h"

namespace csa {

namespace {

constexpr int kAttnThreads = 256;
constexpr int kSplitRows = 32;
constexpr int kHeadGroup = 16;
constexpr int kMaxD = 512;

inline int attn_splits(int n_max) { return n_max > 0 ? (n_max + kSplitRows - 1) / kSplitRows : 1; }

__global__ __launch_bounds__(kAttnThreads) void k_attn_partial_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int* __restrict__ n_valid,
    float scale, int h, int d, int n_max, long long q_stride_b, long long kv_stride_b,
    float* __restrict__ ws_o, float* __restrict__ ws_ml, int n_splits) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[kSplitRows * (kMaxD + 8)];
    __shared__ __attribute__((aligned(16))) uint16_t pl[kHeadGroup * (kSplitRows + 8)];
    __shared__ float spart[4][kHeadGroup][kSplitRows];

    const int split = blockIdx.x;
    const int hg = blockIdx.y;
    const int b = blockIdx.z;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int pitch = d + 8;
    int nv = n_valid[b];
    nv = nv < 0 ? 0 : (nv > n_max ? n_max : nv);
    const int r0 = split * kSplitRows;
    const int rows = max(0, min(kSplitRows, nv - r0));
    const long long ml_base = (static_cast<long long>(b) * h + hg * kHeadGroup) * n_splits + split;

    if (rows == 0) {  // nothing to attend in this split: mark it empty
        if (threadIdx.x < kHeadGroup) {
            ws_ml[2 * (ml_base + static_cast<long long>(threadIdx.x) * n_splits) + 0] = -INFINITY;
            ws_ml[2 * (ml_base + static_cast<long long>(threadIdx.x) * n_splits) + 1] = 0.f;
        }
        return;
    }

    // 1. key/value tile -> LDS (zero rows beyond n_valid so P*V stays finite)
    const int cpr = d / 8;  // 16-byte chunks per row
    const uint16_t* kvb = kv + b * kv_stride_b + static_cast<long long>(r0) * d;
    for (int c = threadIdx.x; c < kSplitRows * cpr; c += kAttnThreads) {
        const int r = c / cpr;
        const int cc = c - r * cpr;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < rows) v = *reinterpret_cast<const uint4*>(kvb + static_cast<long long>(r) * d + cc * 8);
        *reinterpret_cast<uint4*>(tile + r * pitch + cc * 8) = v;
    }
    __syncthreads();

    // 2. S = q K^T: M = 16 heads, N = 2 x 16 rows, K = d split across waves.
    const int li = lane & 15;
    const int lg = lane >> 4;
    const uint16_t* qh = q + b * q_stride_b + static_cast<long long>(hg * kHeadGroup + li) * d + 8 * lg;
    f32x4 s0 = {}, s1 = {};
    for (int ks = wv; ks < d / 32; ks += 4) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(qh + 32 * ks);
        const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(tile + li * pitch + 32 * ks + 8 * lg);
        const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(tile + (16 + li) * pitch + 32 * ks + 8 * lg);
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b0, s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b1, s1, 0, 0, 0);
    }
    // accumulator layout: register r <-> head 4*lg + r, row li (+16 for s1)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        spart[wv][4 * lg + r][li] = s0[r];
        spart[wv][4 * lg + r][16 + li] = s1[r];
    }
    __syncthreads();

    // 3. local softmax: thread -> head hh = tid/16, rows 2*(tid%16) + {0,1}
    {
        const int hh = threadIdx.x >> 4;
        const int j0 = 2 * (threadIdx.x & 15);
        float x0 = (spart[0][hh][j0] + spart[1][hh][j0] + spart[2][hh][j0] + spart[3][hh][j0]) * scale;
        float x1 = (spart[0][hh][j0 + 1] + spart[1][hh][j0 + 1] + spart[2][hh][j0 + 1] + spart[3][hh][j0 + 1]) * scale;
        if (j0 >= rows) x0 = -INFINITY;
        if (j0 + 1 >= rows) x1 = -INFINITY;
        float mx = fmaxf(x0, x1);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        // rows >= 1 here, so mx is finite
        const uint16_t p0 = f32_to_bf16(expf(x0 - mx));
        const uint16_t p1 = f32_to_bf16(expf(x1 - mx));
        float l = bf16_to_f32(p0) + bf16_to_f32(p1);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) l += __shfl_xor(l, o);
        pl[hh * (kSplitRows + 8) + j0] = p0;
        pl[hh * (kSplitRows + 8) + j0 + 1] = p1;
        if ((threadIdx.x & 15) == 0) {
            ws_ml[2 * (ml_base + static_cast<long long>(hh) * n_splits) + 0] = mx;
            ws_ml[2 * (ml_base + static_cast<long long>(hh) * n_splits) + 1] = l;
        }
    }
    __syncthreads();

    // 4. O = P V: M = 16 heads, K = 32 rows (one MFMA step), N = d in 16-wide tiles.
    const bf16x8 pa = *reinterpret_cast<const bf16x8*>(pl + li * (kSplitRows + 8) + 8 * lg);
    float* ob = ws_o + (static_cast<long long>(b) * h + hg * kHeadGroup) * n_splits * d +
                static_cast<long long>(split) * d;
    for (int nt = wv; nt < d / 16; nt += 4) {
        const int col = 16 * nt + li;
        bf16x8 vb;
        uint16_t tmp[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) tmp[e] = tile[(8 * lg + e) * pitch + col];
        __builtin_memcpy(&vb, tmp, sizeof(vb));
        f32x4 o = {};
        o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, o, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            ob[static_cast<long long>(4 * lg + r) * n_splits * d + col] = o[r];
    }
}

__global__ __launch_bounds__(kAttnThreads) void k_attn_merge(const float* __restrict__ ws_o,
                                                             const float* __restrict__ ws_ml,
                                                             const float* __restrict__ sink, int h,
                                                             int d, int n_splits, void* __restrict__ out,
                                                             int out_bf16, float* __restrict__ lse,
                                                             long long out_stride_b) {
    const int hh = blockIdx.x;
    const int b = blockIdx.y;
    const long long base = (static_cast<long long>(b) * h + hh) * n_splits;
    const float* ml = ws_ml + 2 * base;
    float M = sink ? sink[hh] : -INFINITY;
    for (int s = 0; s < n_splits; ++s)
        if (ml[2 * s + 1] > 0.f) M = fmaxf(M, ml[2 * s]);
    float den = 0.f;
    if (M != -INFINITY) {
        for (int s = 0; s < n_splits; ++s)
            if (ml[2 * s + 1] > 0.f) den += ml[2 * s + 1] * expf(ml[2 * s] - M);
        if (sink) den += expf(sink[hh] - M);
    }
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    const float* ob = ws_o + base * d;
    for (int dd = threadIdx.x; dd < d; dd += blockDim.x) {
        float acc = 0.f;
        for (int s = 0; s < n_splits; ++s)
            if (ml[2 * s + 1] > 0.f) acc += ob[static_cast<long long>(s) * d + dd] * expf(ml[2 * s] - M);
        const float y = acc * inv;
        const long long o = b * out_stride_b + static_cast<long long>(hh) * d + dd;
        if (out_bf16) static_cast<uint16_t*>(out)[o] = f32_to_bf16(y);
        else static_cast<float*>(out)[o] = y;
    }
    if (lse && threadIdx.x == 0)
        lse[static_cast<long long>(b) * h + hh] = den > 0.f ? M + logf(den) : -INFINITY;
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

hipError_t launch_attn_bf16(const void* q, const void* kv, const int* n_valid, const float* sink,
                            float scale, void* out, bool out_bf16, float* lse, int batch, int h,
                            int d, int n_max, long long q_stride_b, long long kv_stride_b,
                            long long out_stride_b, void* ws, hipStream_t s) {
    const int ns = attn_splits(n_max);
    float* ws_o = static_cast<float*>(ws);
    float* ws_ml = ws_o + static_cast<size_t>(batch) * h * ns * d;
    hipLaunchKernelGGL(k_attn_partial_bf16, dim3(ns, h / kHeadGroup, batch), dim3(kAttnThreads), 0, s,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv), n_valid,
                       scale, h, d, n_max, q_stride_b, kv_stride_b, ws_o, ws_ml, ns);
    hipLaunchKernelGGL(k_attn_merge, dim3(h, batch), dim3(kAttnThreads), 0, s, ws_o, ws_ml, sink, h,
                       d, ns, out, out_bf16 ? 1 : 0, lse, out_stride_b);
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

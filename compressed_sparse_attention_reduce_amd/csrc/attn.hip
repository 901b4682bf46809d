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
//   k_attn_merge — one workgroup per (head, sequence): M = max(max_s m_s, sink),
//     rescale and add the partials, add exp(sink - M) once, divide.
// float32 path (small correctness workloads): one workgroup per (head,
// sequence), the whole softmax in float32 on the vector ALUs.
#include "common.h"
#include "kernels.h"

namespace csa {

namespace {

constexpr int kAttnThreads = 256;
constexpr int kHeadGroup = 16;

// 32 rows per split: every thread issues all its row loads at once, and
// short rows give more workgroups to spread the loads over.
inline int attn_rows_per_split(int) { return 32; }
inline int attn_splits(int n_max) {
    const int r = attn_rows_per_split(n_max);
    return n_max > 0 ? (n_max + r - 1) / r : 1;
}

template <int R>
__global__ __launch_bounds__(kAttnThreads) void k_attn_partial_bf16(AttnArgs a, int n_splits) {
    constexpr int kNt = R / 16;       // 16-row tiles, one per wave (R = 64) or two waves idle (R = 32)
    constexpr int kPPitch = R + 8;
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    uint16_t* tile = smem;                                   // [R][d + 8]
    uint16_t* qs = tile + R * (a.d + 8);                      // [16][d + 8]
    uint16_t* pl = qs + kHeadGroup * (a.d + 8);               // [16][R + 8]
    __shared__ float wmax[4][kHeadGroup];
    __shared__ float wsum[4][kHeadGroup];

    const int split = blockIdx.x;
    const int hg = blockIdx.y;
    const int b = blockIdx.z;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int d = a.d;
    const int pitch = d + 8;
    const int r0 = split * R;
    const int cpr = d / 8;  // 16-byte chunks per row

    // 0. the query group's loads go first (independent of everything below)
    const uint16_t* qg = a.q + b * a.q_stride_b + static_cast<long long>(hg * kHeadGroup) * d;
    constexpr int kQBatch = kHeadGroup * 64 / kAttnThreads;  // pieces per thread at d = 512
    uint4 qv[kQBatch];
#pragma unroll
    for (int u = 0; u < kQBatch; ++u) {
        const int c = threadIdx.x + u * kAttnThreads;
        qv[u] = c < kHeadGroup * cpr ? *reinterpret_cast<const uint4*>(qg + (c / cpr) * d + (c % cpr) * 8)
                                     : make_uint4(0, 0, 0, 0);
    }

    // valid rows: n_valid from the device (gather mode: top-k count + window).
    // Each thread loads the top-k index of every row its chunks fall in
    // alongside the count, so the row loads below wait for one round trip
    // only (lanes of a wave mostly share a row: one request).
    constexpr int kChunks = R * 64 / kAttnThreads;  // 16-byte chunks per thread at d = 512
    const int n_chunks = R * cpr;
    int my_idx[kChunks];
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
        const int c = u * kAttnThreads + threadIdx.x;
        const int j = r0 + c / cpr;
        my_idx[u] = (a.idx && c < n_chunks && j < a.k) ? a.idx[static_cast<long long>(b) * a.k + j] : 0;
    }
    int cnt = 0, nv;
    if (a.idx) {
        cnt = a.count ? a.count[b] : a.k;
        cnt = cnt < 0 ? 0 : (cnt > a.k ? a.k : cnt);
        if (a.n_comp <= 0) cnt = 0;
        nv = cnt + a.swa_len;
        if (split == 0 && hg == 0 && threadIdx.x == 0 && a.n_valid_out) a.n_valid_out[b] = nv;
    } else {
        nv = a.n_valid[b];
    }
    nv = nv < 0 ? 0 : (nv > a.n_max ? a.n_max : nv);
    const int rows = max(0, min(R, nv - r0));
    const long long ml_base = (static_cast<long long>(b) * a.h + hg * kHeadGroup) * n_splits + split;
    if (rows == 0) {
        if (threadIdx.x < kHeadGroup) {
            a.ws_ml[2 * (ml_base + static_cast<long long>(threadIdx.x) * n_splits) + 0] = -INFINITY;
            a.ws_ml[2 * (ml_base + static_cast<long long>(threadIdx.x) * n_splits) + 1] = 0.f;
        }
        return;
    }

    // 1. every chunk's source (top-k row of the compressed cache, SWA slot, or
    //    the plain kv rows), all loads in one unrolled batch: rows -> LDS (and
    //    gather_buf); query -> LDS
    uint4 v[kChunks];
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
        const int c = u * kAttnThreads + threadIdx.x;
        const int r = c / cpr;
        const int j = r0 + r;
        const uint16_t* src = nullptr;
        if (c < n_chunks && r < rows) {
            if (!a.idx) {
                src = a.kv + b * a.kv_stride_b + static_cast<long long>(j) * d;
            } else if (j < cnt) {
                const int ri = my_idx[u] < 0 ? 0 : (my_idx[u] >= a.n_comp ? a.n_comp - 1 : my_idx[u]);
                src = a.comp_kv + b * a.comp_kv_stride_b + static_cast<long long>(ri) * d;
            } else {
                int slot = (a.swa_head - a.swa_len + (j - cnt)) % a.w;
                if (slot < 0) slot += a.w;
                src = a.swa + b * a.swa_stride_b + static_cast<long long>(slot) * d;
            }
        }
        v[u] = src ? *reinterpret_cast<const uint4*>(src + (c % cpr) * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kQBatch; ++u) {
        const int c = threadIdx.x + u * kAttnThreads;
        if (c < kHeadGroup * cpr) *reinterpret_cast<uint4*>(qs + (c / cpr) * pitch + (c % cpr) * 8) = qv[u];
    }
    const bool write_buf = a.idx && a.gather_buf && hg == 0;
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
        const int c = u * kAttnThreads + threadIdx.x;
        if (c < n_chunks) {
            const int r = c / cpr;
            const int cc = c % cpr;
            *reinterpret_cast<uint4*>(tile + r * pitch + cc * 8) = v[u];
            if (write_buf && r < rows)
                *reinterpret_cast<uint4*>(a.gather_buf + b * a.buf_stride_b + static_cast<long long>(r0 + r) * d + cc * 8) = v[u];
        }
    }
    __syncthreads();

    // 2. S = q K^T: wave wv owns rows 16*wv .. 16*wv+15 (if R allows)
    const int li = lane & 15;
    const int lg = lane >> 4;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    const bool has_tile = wv < kNt;
    if (has_tile) {
        for (int ks = 0; ks < d / 32; ++ks) {
            const bf16x8 qa = *reinterpret_cast<const bf16x8*>(qs + li * pitch + 32 * ks + 8 * lg);
            const bf16x8 kb = *reinterpret_cast<const bf16x8*>(tile + (16 * wv + li) * pitch + 32 * ks + 8 * lg);
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kb, s, 0, 0, 0);
        }
    }
    // accumulator register r <-> head 4*lg + r, row 16*wv + li
    const int my_row = 16 * wv + li;
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = (has_tile && my_row < rows) ? s[r] * a.scale : -INFINITY;
    // 3. split softmax: per-head max and sum over the R rows (lanes, then waves)
    float mx[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float v = x[r];
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, row16_xor(v, o));
        mx[r] = v;
    }
    if (li == 0)
#pragma unroll
        for (int r = 0; r < 4; ++r) wmax[wv][4 * lg + r] = mx[r];
    __syncthreads();
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int hh = 4 * lg + r;
        const float M = fmaxf(fmaxf(wmax[0][hh], wmax[1][hh]), fmaxf(wmax[2][hh], wmax[3][hh]));
        // rows >= 1, so M is finite; masked rows give exp(-inf) = 0
        const uint16_t pb = f32_to_bf16(expf(x[r] - M));
        p[r] = bf16_to_f32(pb);
        if (has_tile) pl[hh * kPPitch + my_row] = pb;
        else if (my_row < R) pl[hh * kPPitch + my_row] = 0;
        float v = p[r];
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) v += row16_xor(v, o);
        if (li == 0) wsum[wv][hh] = has_tile ? v : 0.f;
        mx[r] = M;
    }
    __syncthreads();
    if (threadIdx.x < kHeadGroup) {
        const int hh = threadIdx.x;
        const float M = fmaxf(fmaxf(wmax[0][hh], wmax[1][hh]), fmaxf(wmax[2][hh], wmax[3][hh]));
        const float l = wsum[0][hh] + wsum[1][hh] + wsum[2][hh] + wsum[3][hh];
        a.ws_ml[2 * (ml_base + static_cast<long long>(hh) * n_splits) + 0] = M;
        a.ws_ml[2 * (ml_base + static_cast<long long>(hh) * n_splits) + 1] = l;
    }

    // 4. O = P V: M = 16 heads, K = R rows (R/32 MFMA steps), N = d in 16-wide tiles
    float* ob = a.ws_o + (static_cast<long long>(b) * a.h + hg * kHeadGroup) * n_splits * d +
                static_cast<long long>(split) * d;
    for (int nt = wv; nt < d / 16; nt += 4) {
        const int col = 16 * nt + li;
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < R / 32; ++ks) {
            const bf16x8 pa = *reinterpret_cast<const bf16x8*>(pl + li * kPPitch + 32 * ks + 8 * lg);
            bf16x8 vb;
            uint16_t tmp[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) tmp[e] = tile[(32 * ks + 8 * lg + e) * pitch + col];
            __builtin_memcpy(&vb, tmp, sizeof(vb));
            o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, o, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) ob[static_cast<long long>(4 * lg + r) * n_splits * d + col] = o[r];
    }
}

constexpr int kMaxSplits = 256;

__global__ __launch_bounds__(kAttnThreads) void k_attn_merge(const float* __restrict__ ws_o,
                                                             const float* __restrict__ ws_ml,
                                                             const float* __restrict__ sink, int h,
                                                             int d, int n_splits, void* __restrict__ out,
                                                             int out_bf16, float* __restrict__ lse,
                                                             long long out_stride_b) {
    const int hh = blockIdx.x;
    const int b = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    const long long base = (static_cast<long long>(b) * h + hh) * n_splits;
    const float* ml = ws_ml + 2 * base;
    const float* ob = ws_o + base * d;
    // Partials of empty splits (l = 0) are never written: their loads read
    // stale workspace bytes that are skipped below (never multiplied).
    // Thread t owns columns 2t and 2t + 1; the first splits' loads go first.
    const int col = 2 * threadIdx.x;
    const bool has_col = col < d;
    constexpr int kBatch = 32;  // all splits of a 1024-row window in one round trip
    float2 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
        v[u] = (has_col && u < n_splits) ? *reinterpret_cast<const float2*>(ob + static_cast<long long>(u) * d + col)
                                         : make_float2(0.f, 0.f);
    // split weights, derived by every wave on its own (no barrier): lane s
    // holds split s of each group of 64
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
    float2 acc = make_float2(0.f, 0.f);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
        if (u < n_splits) {
            const float c = coef(u);
            if (c != 0.f) {
                acc.x += v[u].x * c;
                acc.y += v[u].y * c;
            }
        }
    }
    for (int s0 = kBatch; s0 < n_splits; s0 += kBatch) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            v[u] = (has_col && s0 + u < n_splits)
                       ? *reinterpret_cast<const float2*>(ob + static_cast<long long>(s0 + u) * d + col)
                       : make_float2(0.f, 0.f);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (s0 + u < n_splits) {
                const float c = coef(s0 + u);
                if (c != 0.f) {
                    acc.x += v[u].x * c;
                    acc.y += v[u].y * c;
                }
            }
        }
    }
    if (has_col) {
        const long long o = b * out_stride_b + static_cast<long long>(hh) * d + col;
        if (out_bf16) {
            static_cast<uint16_t*>(out)[o] = f32_to_bf16(acc.x);
            static_cast<uint16_t*>(out)[o + 1] = f32_to_bf16(acc.y);
        } else {
            static_cast<float*>(out)[o] = acc.x;
            static_cast<float*>(out)[o + 1] = acc.y;
        }
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

int attn_max_splits() { return kMaxSplits; }

int attn_max_rows() { return kMaxSplits * 32; }

hipError_t launch_attn_bf16(AttnArgs a, hipStream_t s) {
    const int ns = attn_splits(a.n_max);
    const int R = attn_rows_per_split(a.n_max);
    a.ws_o = static_cast<float*>(a.ws);
    a.ws_ml = a.ws_o + static_cast<size_t>(a.batch) * a.h * ns * a.d;
    const size_t lds = sizeof(uint16_t) * (static_cast<size_t>(R + kHeadGroup) * (a.d + 8) + kHeadGroup * (R + 8));
    // above 64 KB of dynamic LDS the kernel must opt in (gfx950 has 160 KB per workgroup), once per device
    {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
        static bool opted_in[64] = {};
        if (!opted_in[dev]) {
            const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_partial_bf16<32>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 1024);
            if (e != hipSuccess) return e;
            opted_in[dev] = true;
        }
    }
    if (R != 32) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_attn_partial_bf16<32>, dim3(ns, a.h / kHeadGroup, a.batch), dim3(kAttnThreads), lds, s, a,
                       ns);
    hipLaunchKernelGGL(k_attn_merge, dim3(a.h, a.batch), dim3(kAttnThreads), 0, s, a.ws_o, a.ws_ml, a.sink, a.h,
                       a.d, ns, a.out, a.out_bf16 ? 1 : 0, a.lse, a.out_stride_b);
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

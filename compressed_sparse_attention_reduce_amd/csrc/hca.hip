// Dense split attention of the HCA layers: one softmax (scale, then the sink
// in the denominator) over every compressed entry followed by the live SWA
// window — page 1, PERFORMANCE_AUDIT.md, the forward_attention branch for
// ratios above 4 (torch.cat([kv_cache.comp_kv, swa_kv])); the sink of the
// D5c hunk (fmha_6warp_tma_multirow_multitile.cuh).
//
// The sparse path's splits hold 32 rows, which suits its 640 rows; at 1M
// context an HCA layer attends to ~7900 rows, and 32-row splits would write
// as many partial bytes as they read.  Here a split is 128 rows held in LDS
// at once (one round of loads, eight waves: one 16-row tile of S = q K^T
// each, then four 16-column tiles of O = P V each, both on
// v_mfma_f32_16x16x32_bf16), so the partials are a quarter of the row bytes
// and the merge (k_attn_merge, shared with the sparse path) reads a quarter
// of the splits.  The four head groups of a split run on one XCD
// (consecutive workgroup ids go to consecutive XCDs), so the rows come from
// HBM once and from that XCD's L2 for the other three groups.
#include "attn_split.h"
#include "common.h"
#include "kernels.h"
#include "step_prep.h"

namespace csa {

namespace {

constexpr int kDenseThreads = 512;
constexpr int kDenseWaves = kDenseThreads / kWave;
constexpr int kDenseRows = 16 * kDenseWaves;          // rows per split: one 16-row S tile per wave
constexpr int kDensePPitch = kDenseRows + 8;          // LDS pitch of the probabilities
constexpr int kDenseMaxD = 512;
constexpr int kDenseQPer = kHeadGroup * kDenseMaxD / 8 / kDenseThreads;  // query pieces per thread
constexpr int kDenseRowPer = kDenseRows * kDenseMaxD / 8 / kDenseThreads; // row pieces per thread

__host__ __device__ inline size_t dense_lds_bytes(int d) {
    return sizeof(uint16_t) * (static_cast<size_t>(kDenseRows + kHeadGroup) * (d + 8) +
                               static_cast<size_t>(kHeadGroup) * kDensePPitch);
}

__global__ __launch_bounds__(kDenseThreads) void k_attn_dense_bf16(AttnArgs a, int n_splits, int prep_wgs, PrepArgs p,
                                                                    int extra_rows) {
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    __shared__ float wmax[kDenseWaves][kHeadGroup];
    __shared__ float wsum[kDenseWaves][kHeadGroup];
    // the step's small jobs (SWA append, compression of a completed block) in
    // their own workgroups; the rows they write are not
    // read here (the attention covers the rows before the step, the merge
    // adds the two new ones)
    // (first in the grid, so they start before the attention fills the CUs)
    if (static_cast<int>(blockIdx.x) < prep_wgs) {
        step_prep_role(p, blockIdx.x, blockIdx.y, reinterpret_cast<float*>(smem), &wmax[0][0]);
        return;
    }
    const int groups = a.h / kHeadGroup;
    // workgroup id -> (split, head group): id % 8 = split % 8, so a split's
    // head groups share an XCD
    const int id = blockIdx.x - prep_wgs;
    const int rest = id / 8;
    const int hg = rest % groups;
    const int split = id % 8 + 8 * (rest / groups);
    const int b = blockIdx.y;
    if (split >= n_splits) return;  // padding of the grid: never merged
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int d = a.d;
    const int pitch = d + 8;
    const int cpr = d / 8;
    uint16_t* tile = smem;                         // [kDenseRows][d + 8]
    uint16_t* qs = tile + kDenseRows * pitch;      // [16][d + 8]
    uint16_t* pl = qs + kHeadGroup * pitch;        // [16][kDenseRows + 8]
    const int cnt = a.n_comp > 0 ? a.n_comp : 0;
    int nv = cnt + a.swa_len;
    nv = nv > a.n_max ? a.n_max : nv;
    const int r0 = split * kDenseRows;
    const int rows = max(0, min(kDenseRows, nv - r0));
    const long long ml_base = (static_cast<long long>(b) * a.h + hg * kHeadGroup) * n_splits + split;
    if (split == 0 && hg == 0 && threadIdx.x == 0 && a.n_valid_out) a.n_valid_out[b] = nv + extra_rows;
    if (rows == 0) {
        if (threadIdx.x < kHeadGroup) {
            a.ws_ml[2 * (ml_base + static_cast<long long>(threadIdx.x) * n_splits) + 0] = -INFINITY;
            a.ws_ml[2 * (ml_base + static_cast<long long>(threadIdx.x) * n_splits) + 1] = 0.f;
        }
        return;
    }
    // 1. query group and the split's rows to LDS, all loads in one batch
    const uint16_t* qg = a.q + b * a.q_stride_b + static_cast<long long>(hg * kHeadGroup) * d;
    const uint16_t* comp = a.comp_kv + b * a.comp_kv_stride_b;
    const uint16_t* swa = a.swa + b * a.swa_stride_b;
    uint4 qv[kDenseQPer], v[kDenseRowPer];
#pragma unroll
    for (int u = 0; u < kDenseQPer; ++u) {
        const int c = threadIdx.x + u * kDenseThreads;
        qv[u] = c < kHeadGroup * cpr ? *reinterpret_cast<const uint4*>(qg + (c / cpr) * d + (c % cpr) * 8)
                                     : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kDenseRowPer; ++u) {
        const int c = threadIdx.x + u * kDenseThreads;
        const int r = c / cpr;
        const int j = r0 + r;
        const uint16_t* src = nullptr;
        if (c < kDenseRows * cpr && r < rows) {
            if (j < cnt) {
                src = comp + static_cast<long long>(j) * d;
            } else {
                int slot = (a.swa_head - a.swa_len + (j - cnt)) % a.w;
                if (slot < 0) slot += a.w;
                src = swa + static_cast<long long>(slot) * d;
            }
        }
        v[u] = src ? *reinterpret_cast<const uint4*>(src + (c % cpr) * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kDenseQPer; ++u) {
        const int c = threadIdx.x + u * kDenseThreads;
        if (c < kHeadGroup * cpr) *reinterpret_cast<uint4*>(qs + (c / cpr) * pitch + (c % cpr) * 8) = qv[u];
    }
#pragma unroll
    for (int u = 0; u < kDenseRowPer; ++u) {
        const int c = threadIdx.x + u * kDenseThreads;
        if (c < kDenseRows * cpr) *reinterpret_cast<uint4*>(tile + (c / cpr) * pitch + (c % cpr) * 8) = v[u];
    }
    __syncthreads();

    // 2. S = q K^T: wave wv owns rows 16*wv .. 16*wv+15; per-head max of the wave
    const int my_row = 16 * wv + li;
    float x[4];
    {
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
        const uint16_t* qrow = qs + li * pitch + 8 * lg;
        const uint16_t* krow = tile + my_row * pitch + 8 * lg;
        const int nks = d / 32;
        int ks = 0;
        for (; ks + 4 <= nks; ks += 4) {
            bf16x8 qa[4], kb[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                qa[u] = *reinterpret_cast<const bf16x8*>(qrow + 32 * (ks + u));
                kb[u] = *reinterpret_cast<const bf16x8*>(krow + 32 * (ks + u));
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[u], kb[u], sacc, 0, 0, 0);
        }
        for (; ks < nks; ++ks)
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(qrow + 32 * ks),
                                                           *reinterpret_cast<const bf16x8*>(krow + 32 * ks), sacc,
                                                           0, 0, 0);
        // accumulator register r <-> head 4*lg + r, row my_row
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            x[r] = my_row < rows ? sacc[r] * a.scale : -INFINITY;
            float mx = x[r];
#pragma unroll
            for (int q = 1; q < 16; q <<= 1) mx = fmaxf(mx, row16_xor(mx, q));
            if (li == 0) wmax[wv][4 * lg + r] = mx;
        }
    }
    __syncthreads();
    // 3. probabilities against the split's max (finite: row 0 is valid)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int hh = 4 * lg + r;
        float M = wmax[0][hh];
#pragma unroll
        for (int w = 1; w < kDenseWaves; ++w) M = fmaxf(M, wmax[w][hh]);
        const uint16_t pb = f32_to_bf16(expf(x[r] - M));
        pl[hh * kDensePPitch + my_row] = pb;
        float e = bf16_to_f32(pb);
#pragma unroll
        for (int q = 1; q < 16; q <<= 1) e += row16_xor(e, q);
        if (li == 0) wsum[wv][hh] = e;
    }
    __syncthreads();
    if (threadIdx.x < kHeadGroup) {
        const int hh = threadIdx.x;
        float M = wmax[0][hh], l = wsum[0][hh];
#pragma unroll
        for (int w = 1; w < kDenseWaves; ++w) {
            M = fmaxf(M, wmax[w][hh]);
            l += wsum[w][hh];
        }
        a.ws_ml[2 * (ml_base + static_cast<long long>(hh) * n_splits) + 0] = M;
        a.ws_ml[2 * (ml_base + static_cast<long long>(hh) * n_splits) + 1] = l;
    }
    // 4. O = P V: M = 16 heads, K = the split's rows in 32-row steps, N = d in 16-wide tiles
    float* ob = a.ws_o + (static_cast<long long>(b) * a.h + hg * kHeadGroup) * n_splits * d +
                static_cast<long long>(split) * d;
    const int ksteps = (rows + 31) / 32;  // rows past the valid ones hold zeros and p = 0
    for (int nt = wv; nt < d / 16; nt += kDenseWaves) {
        const int col = 16 * nt + li;
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
        for (int ks = 0; ks < ksteps; ++ks) {
            const bf16x8 pa = *reinterpret_cast<const bf16x8*>(pl + li * kDensePPitch + 32 * ks + 8 * lg);
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

// Merge of the splits plus the step's new rows (the compressed entry of a
// completed block, x0, if any; the new token's KV row, x1), one workgroup per
// (head, sequence): M = max of the splits' maxima, the new rows' logits and
// the sink; out = (sum_s e^(m_s - M) O_s + sum_i e^(s_i - M) x_i) / den with
// den = sum_s e^(m_s - M) l_s + sum_i e^(s_i - M) + e^(sink - M).  At most
// 64 splits (lane s of every wave holds split s's (m, l)).
constexpr int kMergeThreads = 256;
__global__ __launch_bounds__(kMergeThreads) void k_attn_merge_rows(AttnArgs a, int n_splits, const uint16_t* x0,
                                                                   long long x0_stride_b, const uint16_t* x1,
                                                                   long long x1_stride_b) {
    __shared__ float red[2][kMergeThreads / kWave];
    const int hh = blockIdx.x;
    const int b = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int d = a.d;
    const long long base = (static_cast<long long>(b) * a.h + hh) * n_splits;
    const float* ob = a.ws_o + base * d;
    const int col = 2 * threadIdx.x;
    const bool has_col = col < d;
    // the new rows' logits: q . x_i over the block, two sums at once
    const uint16_t* qh = a.q + b * a.q_stride_b + static_cast<long long>(hh) * d;
    float q0 = 0.f, q1 = 0.f, a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
    if (has_col) {
        const uint32_t qq = *reinterpret_cast<const uint32_t*>(qh + col);
        q0 = __uint_as_float(qq << 16);
        q1 = __uint_as_float(qq & 0xffff0000u);
        if (x0) {
            const uint32_t xx = *reinterpret_cast<const uint32_t*>(x0 + b * x0_stride_b + col);
            a0 = __uint_as_float(xx << 16);
            a1 = __uint_as_float(xx & 0xffff0000u);
        }
        const uint32_t yy = *reinterpret_cast<const uint32_t*>(x1 + b * x1_stride_b + col);
        b0 = __uint_as_float(yy << 16);
        b1 = __uint_as_float(yy & 0xffff0000u);
    }
    float d0 = wave_sum(q0 * a0 + q1 * a1);
    float d1 = wave_sum(q0 * b0 + q1 * b1);
    if (lane == 0) {
        red[0][wv] = d0;
        red[1][wv] = d1;
    }
    __syncthreads();
    d0 = 0.f;
    d1 = 0.f;
#pragma unroll
    for (int w = 0; w < kMergeThreads / kWave; ++w) {
        d0 += red[0][w];
        d1 += red[1][w];
    }
    const float s0 = x0 ? d0 * a.scale : -INFINITY;
    const float s1 = d1 * a.scale;
    // split weights
    const float ms = lane < n_splits ? a.ws_ml[2 * (base + lane)] : -INFINITY;
    const float ls = lane < n_splits ? a.ws_ml[2 * (base + lane) + 1] : 0.f;
    float M = wave_max(ls > 0.f ? ms : -INFINITY);
    M = fmaxf(M, fmaxf(s0, s1));
    const float sk = a.sink ? a.sink[hh] : -INFINITY;
    M = fmaxf(M, sk);  // finite: s1 is
    const float wsp = ls > 0.f ? expf(ms - M) : 0.f;
    const float e0 = x0 ? expf(s0 - M) : 0.f;
    const float e1 = expf(s1 - M);
    const float es = a.sink ? expf(sk - M) : 0.f;
    const float den = wave_sum(wsp * ls) + e0 + e1 + es;
    const float inv = 1.0f / den;
    float acc0 = e0 * a0 + e1 * b0, acc1 = e0 * a1 + e1 * b1;
    // the splits' outputs in batches of loads; empty splits' slots hold stale
    // bytes, selected away (never multiplied)
    constexpr int kBatch = 16;
    for (int s0b = 0; s0b < n_splits; s0b += kBatch) {
        float2 v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            v[u] = (has_col && s0b + u < n_splits)
                       ? *reinterpret_cast<const float2*>(ob + static_cast<long long>(s0b + u) * d + col)
                       : make_float2(0.f, 0.f);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int sp = s0b + u < n_splits ? s0b + u : 0;
            const float c = s0b + u < n_splits ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wsp), sp)) : 0.f;
            acc0 += c != 0.f ? c * v[u].x : 0.f;
            acc1 += c != 0.f ? c * v[u].y : 0.f;
        }
    }
    if (has_col) {
        const long long o = b * a.out_stride_b + static_cast<long long>(hh) * d + col;
        if (a.out_bf16) {
            static_cast<uint16_t*>(a.out)[o] = f32_to_bf16(acc0 * inv);
            static_cast<uint16_t*>(a.out)[o + 1] = f32_to_bf16(acc1 * inv);
        } else {
            static_cast<float*>(a.out)[o] = acc0 * inv;
            static_cast<float*>(a.out)[o + 1] = acc1 * inv;
        }
    }
    if (a.lse && threadIdx.x == 0) a.lse[static_cast<long long>(b) * a.h + hh] = M + logf(den);
}

}  // namespace

int attn_dense_splits(int n_max) { return n_max > 0 ? (n_max + kDenseRows - 1) / kDenseRows : 1; }

hipError_t launch_attn_dense_bf16(AttnArgs a, const PrepArgs& prep, const void* x0, long long x0_stride_b,
                                  const void* x1, long long x1_stride_b, hipStream_t s) {
    if (a.d > kDenseMaxD || a.d % 32 != 0 || a.h % kHeadGroup != 0 || !x1) return hipErrorInvalidValue;
    const int ns = attn_dense_splits(a.n_max);
    if (ns > kWave) return hipErrorInvalidValue;
    a.ws_o = static_cast<float*>(a.ws);
    a.ws_ml = a.ws_o + static_cast<size_t>(a.batch) * a.h * ns * a.d;
    const size_t lds = dense_lds_bytes(a.d);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    static bool opted[64] = {};
    if (!opted[dev]) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_dense_bf16),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(dense_lds_bytes(kDenseMaxD)));
        if (e != hipSuccess) return e;
        opted[dev] = true;
    }
    const int groups = a.h / kHeadGroup;
    const int att_wgs = 8 * groups * ((ns + 7) / 8);
    const int prep_wgs = !prep.completes ? 1 : (prep.main_wgs > 1 ? 1 + prep.main_wgs : 2);
    const int extra = 1 + (x0 ? 1 : 0);
    hipLaunchKernelGGL(k_attn_dense_bf16, dim3(att_wgs + prep_wgs, a.batch), dim3(kDenseThreads), lds, s, a, ns,
                       prep_wgs, prep, extra);
    hipLaunchKernelGGL(k_attn_merge_rows, dim3(a.h, a.batch), dim3(kMergeThreads), 0, s, a, ns,
                       static_cast<const uint16_t*>(x0), x0_stride_b, static_cast<const uint16_t*>(x1), x1_stride_b);
    return hipGetLastError();
}

}  // namespace csa

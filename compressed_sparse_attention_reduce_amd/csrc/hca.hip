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

__global__ __launch_bounds__(kDenseThreads) void k_attn_dense_bf16(AttnArgs a, int n_splits) {
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    __shared__ float wmax[kDenseWaves][kHeadGroup];
    __shared__ float wsum[kDenseWaves][kHeadGroup];
    const int groups = a.h / kHeadGroup;
    // workgroup id -> (split, head group): id % 8 = split % 8, so a split's
    // head groups share an XCD
    const int id = blockIdx.x;
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
    if (split == 0 && hg == 0 && threadIdx.x == 0 && a.n_valid_out) a.n_valid_out[b] = nv;
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

}  // namespace

int attn_dense_splits(int n_max) { return n_max > 0 ? (n_max + kDenseRows - 1) / kDenseRows : 1; }

hipError_t launch_attn_dense_bf16(AttnArgs a, hipStream_t s) {
    if (a.d > kDenseMaxD || a.d % 32 != 0 || a.h % kHeadGroup != 0) return hipErrorInvalidValue;
    const int ns = attn_dense_splits(a.n_max);
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
    const int wgs = 8 * groups * ((ns + 7) / 8);
    hipLaunchKernelGGL(k_attn_dense_bf16, dim3(wgs, a.batch), dim3(kDenseThreads), lds, s, a, ns);
    return launch_attn_merge(a, ns, s);
}

}  // namespace csa

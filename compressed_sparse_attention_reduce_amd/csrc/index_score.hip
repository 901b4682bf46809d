// Lightning-indexer score: I[t,s] = sum_h w[t,h] * ReLU(q[t,h] . K[s]).
//
// Page 1, ARCHITECTURE_AND_MEMORY_AUDIT.md, finding F3 (paper section 2.3.1,
// eq. 16): one d_i = 128 key per compressed block, shared by all 64 indexer
// heads (MQA).  Causal form: page 1, archived_plans/NEXT_STEPS.md, Issue 2.
//
// bf16 path (the decode hot spot, HBM-bound at 64 FLOP per key byte):
//   * each wave keeps the query (64 heads x 128 = 16 KB) resident in VGPRs as
//     the A operand of v_mfma_f32_32x32x16_bf16 (heads = M, two 32-row tiles);
//   * key tiles of 32 blocks stream straight from HBM into B-operand VGPRs
//     (each lane loads 16 contiguous bytes of one key row; lanes l and l+32
//     cover 32 contiguous bytes of the same row per k-step), one tile ahead;
//   * the epilogue applies ReLU and the head weights in registers — every lane
//     holds 32 heads of one key — and finishes the head sum with one lane
//     swap (l <-> l+32), so scores leave as one coalesced 128 B store per tile;
//   * optionally it also builds the 12-bit radix histogram of the scores that
//     the top-k filter uses (LDS atomics, flushed once per workgroup).
// Workgroups own contiguous key ranges of one query row; the grid is sized to
// fill every CU with two 4-wave workgroups.
#include "common.h"
#include "kernels.h"

namespace csa {

namespace {

constexpr int kScoreThreads = 256;
constexpr int kWavesPerWg = kScoreThreads / kWave;
constexpr int kTileKeys = 32;
constexpr int kHeads = 64;
constexpr int kDi = 128;
constexpr int kSteps = kDi / 16;  // k-steps of the 32x32x16 MFMA

template <bool kHist>
__global__ __launch_bounds__(kScoreThreads, 2) void k_index_score_bf16(ScoreArgs a,
                                                                       int tiles_per_row,
                                                                       int tiles_per_wg) {
    __shared__ uint32_t lhist[kHist ? kHistBins : 1];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int row = blockIdx.y;
    const int b = row / a.t;
    const int tt = row - b * a.t;
    const int tile0 = blockIdx.x * tiles_per_wg;
    const int tile1 = min(tile0 + tiles_per_wg, tiles_per_row);
    const int hi = lane & 31;   // M row (head) of the A operand / N column (key) of B
    const int grp = lane >> 5;  // which 8-element half of each 16-wide k-step

    if (kHist) {
        for (int i = threadIdx.x; i < kHistBins; i += kScoreThreads) lhist[i] = 0;
        __syncthreads();
    }

    // A operand: q[head][16*s + 8*grp + e] for heads hi and 32 + hi.
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + b * a.q_stride_b +
                           static_cast<long long>(tt) * kHeads * kDi;
    bf16x8 qa0[kSteps], qa1[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        qa0[s] = *reinterpret_cast<const bf16x8*>(qrow + hi * kDi + 16 * s + 8 * grp);
        qa1[s] = *reinterpret_cast<const bf16x8*>(qrow + (32 + hi) * kDi + 16 * s + 8 * grp);
    }
    // Head weights for the 16 accumulator rows this lane holds in each M tile:
    // register r <-> head 8*(r/4) + 4*grp + (r%4).
    const float* wrow = a.w + b * a.w_stride_b + static_cast<long long>(tt) * kHeads;
    float w0[16], w1[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        const float4 v0 = *reinterpret_cast<const float4*>(wrow + 8 * q4 + 4 * grp);
        const float4 v1 = *reinterpret_cast<const float4*>(wrow + 32 + 8 * q4 + 4 * grp);
        w0[4 * q4 + 0] = v0.x; w0[4 * q4 + 1] = v0.y; w0[4 * q4 + 2] = v0.z; w0[4 * q4 + 3] = v0.w;
        w1[4 * q4 + 0] = v1.x; w1[4 * q4 + 1] = v1.y; w1[4 * q4 + 2] = v1.z; w1[4 * q4 + 3] = v1.w;
    }

    const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + b * a.k_stride_b;
    float* srow = a.scores + b * a.s_stride_b + static_cast<long long>(tt) * a.ld_s;
    const long long pos = a.q_pos ? static_cast<long long>(a.q_pos[row]) : 0;
    const int n = a.n;

    auto load_tile = [&](int tile, bf16x8* dst) {
        const int key = min(tile * kTileKeys + hi, n - 1);  // tail lanes re-read a valid row
        const uint16_t* p = kbase + static_cast<long long>(key) * kDi + 8 * grp;
#pragma unroll
        for (int s = 0; s < kSteps; ++s) dst[s] = *reinterpret_cast<const bf16x8*>(p + 16 * s);
    };

    int tile = tile0 + wv;
    bf16x8 kb[kSteps];
    if (tile < tile1) load_tile(tile, kb);
    for (; tile < tile1; tile += kWavesPerWg) {
        bf16x8 kn[kSteps];
        const int nxt = tile + kWavesPerWg;
        if (nxt < tile1) load_tile(nxt, kn);

        f32x16 acc0 = {}, acc1 = {};
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa0[s], kb[s], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa1[s], kb[s], acc1, 0, 0, 0);
        }
        float part = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            part += w0[r] * fmaxf(acc0[r], 0.f);
            part += w1[r] * fmaxf(acc1[r], 0.f);
        }
        part += __shfl_xor(part, 32);

        const int key = tile * kTileKeys + hi;
        if (grp == 0 && key < n) {
            float sc = part;
            if (a.q_pos && static_cast<long long>(a.ratio) * key + a.ratio - 1 > pos) sc = -INFINITY;
            srow[key] = sc;
            if (kHist) {
                const uint32_t kk = score_key(sc);
                if (key_valid(kk, sc)) atomicAdd(&lhist[kk >> (32 - kHistBits)], 1u);
            }
        }
#pragma unroll
        for (int s = 0; s < kSteps; ++s) kb[s] = kn[s];
    }

    if (kHist) {
        __syncthreads();
        uint32_t* gh = a.hist + static_cast<long long>(row) * kHistBins;
        for (int i = threadIdx.x; i < kHistBins; i += kScoreThreads) {
            const uint32_t v = lhist[i];
            if (v) atomicAdd(gh + i, v);
        }
    }
}

// float32 path (small correctness workloads): one thread per key, the query
// and head weights staged in LDS and read as broadcasts.
constexpr int kScoreF32Threads = 256;

__global__ __launch_bounds__(kScoreF32Threads) void k_index_score_f32(ScoreArgs a) {
    extern __shared__ float qs[];  // [h_i * d_i] query, then [h_i] weights
    const int row = blockIdx.y;
    const int b = row / a.t;
    const int tt = row - b * a.t;
    const int hd = a.h_i * a.d_i;
    const float* qrow = static_cast<const float*>(a.q) + b * a.q_stride_b + static_cast<long long>(tt) * hd;
    const float* wrow = a.w + b * a.w_stride_b + static_cast<long long>(tt) * a.h_i;
    for (int i = threadIdx.x; i < hd; i += blockDim.x) qs[i] = qrow[i];
    for (int i = threadIdx.x; i < a.h_i; i += blockDim.x) qs[hd + i] = wrow[i];
    __syncthreads();
    const int key = blockIdx.x * blockDim.x + threadIdx.x;
    if (key >= a.n) return;
    const float* kr = static_cast<const float*>(a.k) + b * a.k_stride_b + static_cast<long long>(key) * a.d_i;
    float sc = 0.f;
    for (int h = 0; h < a.h_i; ++h) {
        float dot = 0.f;
        for (int d = 0; d < a.d_i; ++d) dot += qs[h * a.d_i + d] * kr[d];
        sc += qs[hd + h] * fmaxf(dot, 0.f);
    }
    if (a.q_pos && static_cast<long long>(a.ratio) * key + a.ratio - 1 > a.q_pos[row]) sc = -INFINITY;
    a.scores[b * a.s_stride_b + static_cast<long long>(tt) * a.ld_s + key] = sc;
    if (a.hist) {
        const uint32_t kk = score_key(sc);
        if (key_valid(kk, sc))
            atomicAdd(a.hist + static_cast<long long>(row) * kHistBins + (kk >> (32 - kHistBits)), 1u);
    }
}

}  // namespace

hipError_t launch_index_score_bf16(const ScoreArgs& a, hipStream_t s) {
    if (a.n == 0) return hipSuccess;
    const int rows = a.batch * a.t;
    const int tiles = (a.n + kTileKeys - 1) / kTileKeys;
    const int target = 2 * device_cu_count();
    int wgs = (target + rows - 1) / rows;
    const int max_wgs = (tiles + kWavesPerWg - 1) / kWavesPerWg;
    if (wgs > max_wgs) wgs = max_wgs;
    if (wgs < 1) wgs = 1;
    int per = (tiles + wgs - 1) / wgs;
    per = (per + kWavesPerWg - 1) / kWavesPerWg * kWavesPerWg;
    wgs = (tiles + per - 1) / per;
    if (a.hist)
        hipLaunchKernelGGL(k_index_score_bf16<true>, dim3(wgs, rows), dim3(kScoreThreads), 0, s, a,
                           tiles, per);
    else
        hipLaunchKernelGGL(k_index_score_bf16<false>, dim3(wgs, rows), dim3(kScoreThreads), 0, s, a,
                           tiles, per);
    return hipGetLastError();
}

hipError_t launch_index_score_f32(const ScoreArgs& a, hipStream_t s) {
    if (a.n == 0) return hipSuccess;
    const int rows = a.batch * a.t;
    const size_t lds = sizeof(float) * (static_cast<size_t>(a.h_i) * a.d_i + a.h_i);
    hipLaunchKernelGGL(k_index_score_f32, dim3((a.n + kScoreF32Threads - 1) / kScoreF32Threads, rows),
                       dim3(kScoreF32Threads), lds, s, a);
    return hipGetLastError();
}

}  // namespace csa

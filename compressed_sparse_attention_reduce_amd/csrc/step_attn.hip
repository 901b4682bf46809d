// Fused top-k + partial attention of the bf16 decode step.
//
// Cross-workgroup synchronisation inside a kernel costs a device-scope
// fence per workgroup on this chip (a release fence and a ticket per
// workgroup for the last one to read: about 15 us more per launch at 80
// workgroups, measured with csa_handoff_probe), so instead of a separate
// top-k launch feeding the attention, every
// attention workgroup computes the same (deterministic) top k of its
// sequence from the per-slot candidate lists into LDS, then attends over its
// split of the selected rows plus the SWA window.  Workgroup (0, 0) of each
// sequence also writes topk_idx and topk_count.  Top-k: topk.hip (page 1,
// ARCHITECTURE_AND_MEMORY_AUDIT.md F3); attention: attn.hip (page 1, fmha
// sink correction).  The split partials are merged by k_attn_merge.
#include "attn_split.h"
#include "score_tile.h"
#include "topk_final.h"

namespace csa {

namespace {

__host__ __device__ inline size_t topk_attn_lds_bytes() {
    return sizeof(FinalSmem) + sizeof(int) * kTopkMaxK;
}

__global__ __launch_bounds__(kFinalThreads) void k_topk_attn(TopkArgs ta, CandArgs c, AttnArgs a, int n_splits) {
    if (a.dev)  // counters on the device: the step's view of them after its jobs
        ta.n = attn_dev_view(a, blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0);
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    FinalSmem& fs = *reinterpret_cast<FinalSmem*>(smem);
    int* sidx = reinterpret_cast<int*>(smem + sizeof(FinalSmem));  // this sequence's top-k indices
    const int split = blockIdx.x;
    const int hg = blockIdx.y;
    const int b = blockIdx.z;
    uint4 qv[AttnSplit<kFinalThreads>::kQBatch];
    attn_load_q<kFinalThreads>(a, hg, b, qv);
    // the top k of sequence b (one query row each)
    uint32_t k_eff = 0;
    const bool done = c.lists && union_topk(fs, c, b, ta.k, sidx, k_eff);
    if (!done) {
        __syncthreads();  // the fast path's reads of LDS are over
        k_eff = row_topk(fs, c, b, score_row(ta, b), ta.n, ta.k, sidx);
    }
    __syncthreads();  // sidx complete; the top-k LDS is free for the attention
    if (split == 0 && hg == 0) {
        int* out = ta.idx + static_cast<long long>(b) * ta.k;
        for (int j = threadIdx.x; j < ta.k; j += kFinalThreads) out[j] = j < static_cast<int>(k_eff) ? sidx[j] : -1;
        if (ta.count && threadIdx.x == 0) ta.count[b] = static_cast<int>(k_eff);
    }
    attn_split<kFinalThreads>(a, n_splits, split, hg, b, sidx, static_cast<int>(k_eff), qv,
                              reinterpret_cast<uint16_t*>(smem));
}

static_assert(sizeof(FinalSmem) >= sizeof(uint16_t) * ((kR + kHeadGroup) * (512 + 8) + kHeadGroup * kPPitch),
              "the attention split fits in the top-k LDS at d = 512");

// The two-stage E4M3 selection: every workgroup of sequence b finds the same
// k_cand best by E4M3 score, then workgroup x gives candidates [64 x, 64 x +
// 64) their exact scores: waves 0..3 take 16 candidates each as one B tile
// of v_mfma_f32_16x16x32_bf16 against the bfloat16 query (heads as M) and
// finish with the bfloat16 scan's epilogue (tile_head_sum), so a candidate's
// exact score is the one the bfloat16 step computes for that key.
constexpr int kRescorePerWg = 64;
__global__ __launch_bounds__(kFinalThreads) void k_fp8_rescore(TopkArgs ta, CandArgs c, RescoreArgs r) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    FinalSmem& fs = *reinterpret_cast<FinalSmem*>(smem);
    int* sidx = reinterpret_cast<int*>(smem + sizeof(FinalSmem));
    const int b = blockIdx.y;
    const int kc = ta.k;
    uint32_t k_eff = 0;
    const bool done = c.lists && union_topk(fs, c, b, kc, sidx, k_eff);
    if (!done) {
        __syncthreads();
        k_eff = row_topk(fs, c, b, score_row(ta, b), ta.n, kc, sidx);
    }
    __syncthreads();  // sidx complete
    unsigned long long* out = r.out + static_cast<long long>(b) * (kc + 1);
    if (blockIdx.x == 0 && threadIdx.x == 0) out[kc] = 0ull;  // nothing left out of the list
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    if (wv >= kRescorePerWg / 16) return;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int j = blockIdx.x * kRescorePerWg + 16 * wv + li;  // this lane's candidate (key column li)
    if (blockIdx.x * kRescorePerWg + 16 * wv >= kc) return;   // wave-uniform: past the list
    if (r.n <= 0) {  // no keys: an empty list
        if (lg == 0 && j < kc) out[j] = 0ull;
        return;
    }
    const bool live = j < static_cast<int>(k_eff);
    int key = live ? sidx[j] : 0;
    key = key < 0 ? 0 : (key >= r.n ? r.n - 1 : key);
    const uint16_t* kp = r.keys + b * r.keys_stride_b + static_cast<long long>(key) * 128 + 8 * lg;
    const uint16_t* qb = r.q + b * r.q_stride_b;
    bf16x8 kb[4], qa[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s) kb[s] = *reinterpret_cast<const bf16x8*>(kp + 32 * s);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            qa[mt][s] = *reinterpret_cast<const bf16x8*>(qb + (16 * mt + li) * 128 + 32 * s + 8 * lg);
    float wr[4][4];
    const float* wb = r.w + b * r.w_stride_b;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q) wr[mt][q] = wb[16 * mt + 4 * lg + q];
    f32x4 acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][s], kb[s], acc[mt], 0, 0, 0);
    const float sc = tile_head_sum(acc, wr);
    const uint32_t kk = score_key(sc);
    if (lg == 0 && j < kc) out[j] = (live && key_valid(kk, sc)) ? composite(kk, static_cast<uint32_t>(key)) : 0ull;
}

// The two-stage E4M3 selection of a prefill chunk, one workgroup per query
// row r: the exact scores of its first-stage candidates cand[r][0 .. cnt)
// (bfloat16 query row and keys, the bfloat16 scan's arithmetic: 16
// candidates per wave tile), then the top k of them, sorted.
__global__ __launch_bounds__(kFinalThreads) void k_rescore_rows(RescoreRowsArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    FinalSmem& fs = *reinterpret_cast<FinalSmem*>(smem);
    const int r = blockIdx.x;
    int cnt = a.cand_count ? a.cand_count[r] : a.kc;
    cnt = cnt < 0 ? 0 : (cnt > a.kc ? a.kc : cnt);
    if (a.n <= 0) cnt = 0;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int* cand = a.cand + static_cast<long long>(r) * a.kc;
    const uint16_t* qb = a.q + static_cast<long long>(r) * 64 * 128;
    const float* wb = a.w + static_cast<long long>(r) * 64;
    const int tiles = (cnt + 15) / 16;
    if (wv < tiles) {  // wave-uniform
        bf16x8 qa[4][4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                qa[mt][s] = *reinterpret_cast<const bf16x8*>(qb + (16 * mt + li) * 128 + 32 * s + 8 * lg);
        float wr[4][4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int q = 0; q < 4; ++q) wr[mt][q] = wb[16 * mt + 4 * lg + q];
        for (int tile = wv; tile < tiles; tile += kFinalThreads / kWave) {
            const int j = 16 * tile + li;
            const bool live = j < cnt;
            int key = live ? cand[j] : 0;
            key = key < 0 ? 0 : (key >= a.n ? a.n - 1 : key);
            const uint16_t* kp = a.keys + static_cast<long long>(key) * 128 + 8 * lg;
            bf16x8 kb[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) kb[s] = *reinterpret_cast<const bf16x8*>(kp + 32 * s);
            f32x4 acc[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][s], kb[s], acc[mt], 0, 0, 0);
            const float sc = tile_head_sum(acc, wr);
            if (lg == 0 && live) fs.pool[j] = composite(score_key(sc), static_cast<uint32_t>(key));
        }
    }
    __syncthreads();
    // the top k of the cnt candidates (every composite nonzero: finite scores by contract)
    u64 hi = 0, lo_c = 0;
    for (int i = threadIdx.x; i < cnt; i += kFinalThreads) {
        hi = umax64(hi, fs.pool[i]);
        lo_c = umax64(lo_c, ~fs.pool[i]);
    }
    block_max2(fs, hi, lo_c);
    const int pb = cnt <= 1 ? 0 : __clzll(static_cast<long long>(hi ^ ~lo_c));
    int* out = a.idx + static_cast<long long>(r) * a.k;
    const uint32_t k_eff = cnt > 0 ? select_sorted<kUnionRegs>(fs.pool, static_cast<uint32_t>(cnt),
                                                                static_cast<uint32_t>(a.k), pb, out, fs.stage, fs.ss,
                                                                &fs.n_pool)
                                   : 0u;
    for (int j = static_cast<int>(k_eff) + threadIdx.x; j < a.k; j += kFinalThreads) out[j] = -1;
    if (a.count && threadIdx.x == 0) a.count[r] = static_cast<int>(k_eff);
}

}  // namespace

hipError_t launch_rescore_rows(const RescoreRowsArgs& a, hipStream_t s) {
    if (a.t <= 0) return hipSuccess;
    if (a.kc < 1 || a.kc > kTopkMaxK || a.k < 1 || a.k > a.kc) return hipErrorInvalidValue;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    static bool opted_in[64] = {};
    if (!opted_in[dev]) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_rescore_rows),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(sizeof(FinalSmem)));
        if (e != hipSuccess) return e;
        opted_in[dev] = true;
    }
    hipLaunchKernelGGL(k_rescore_rows, dim3(a.t), dim3(kFinalThreads), sizeof(FinalSmem), s, a);
    return hipGetLastError();
}

hipError_t launch_fp8_rescore(const TopkArgs& ta, const CandArgs* cands, const RescoreArgs& r, hipStream_t s) {
    if (ta.t != 1 || ta.k < 1 || ta.k > kTopkMaxK) return hipErrorInvalidValue;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    static bool opted_in[64] = {};
    if (!opted_in[dev]) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_fp8_rescore),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(topk_attn_lds_bytes()));
        if (e != hipSuccess) return e;
        opted_in[dev] = true;
    }
    const CandArgs c = cands ? *cands : CandArgs{nullptr, 0, 0, 0};
    const int wgs = (ta.k + kRescorePerWg - 1) / kRescorePerWg;
    hipLaunchKernelGGL(k_fp8_rescore, dim3(wgs, ta.batch), dim3(kFinalThreads), topk_attn_lds_bytes(), s, ta, c, r);
    return hipGetLastError();
}

int topk_attn_workgroups(int batch, int h, int n_max) { return attn_splits(n_max) * (h / kHeadGroup) * batch; }

hipError_t launch_topk_attn(const TopkArgs& ta, const CandArgs* cands, AttnArgs a, hipStream_t s) {
    if (ta.t != 1 || a.d > 512 || a.batch != ta.batch) return hipErrorInvalidValue;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    static bool opted_in[64] = {};
    if (!opted_in[dev]) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_topk_attn),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(topk_attn_lds_bytes()));
        if (e != hipSuccess) return e;
        opted_in[dev] = true;
    }
    const int ns = attn_splits(a.n_max);
    a.ws_o = static_cast<float*>(a.ws);
    a.ws_ml = a.ws_o + static_cast<size_t>(a.batch) * a.h * ns * a.d;
    const CandArgs c = cands ? *cands : CandArgs{nullptr, 0, 0, 0};
    hipLaunchKernelGGL(k_topk_attn, dim3(ns, a.h / kHeadGroup, a.batch), dim3(kFinalThreads), topk_attn_lds_bytes(),
                       s, ta, c, a, ns);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_attn_merge(a, ns, s);
}

}  // namespace csa

// Lightning-indexer score: I[t,s] = sum_h w[t,h] * ReLU(q[t,h] . K[s]).
//
// Page 1, ARCHITECTURE_AND_MEMORY_AUDIT.md, finding F3 (paper section 2.3.1,
// eq. 16): one d_i = 128 key per compressed block, shared by all 64 indexer
// heads (MQA).  Causal form: page 1, archived_plans/NEXT_STEPS.md, Issue 2.
//
// bf16 path (the decode hot spot; 64 FLOP per key byte, so HBM-bound on the
// matrix cores):
//   * v_mfma_f32_16x16x32_bf16 with heads as M (4 tiles of 16) and keys as N
//     (tiles of 16 blocks); the query (64 x 128) is staged once per workgroup
//     through LDS into A-operand VGPRs and stays there;
//   * every wave owns an interleaved set of key tiles and keeps a ring of
//     kRing tiles in flight: each lane loads 16 contiguous bytes of one key
//     row per k-step straight into B-operand VGPRs (one instruction covers 16
//     rows x 64 B), and a tile's slot is refilled right after it is consumed,
//     so HBM latency is covered by kRing tiles per wave;
//   * the epilogue applies ReLU and the head weights in registers (each lane
//     holds 16 heads of one key) and finishes the head sum with two lane
//     swaps; 16 scores leave per tile as one 64 B store;
//   * with candidate lists every lane also keeps a short sorted list of its
//     best (score, index) composites in registers (lane group g takes the
//     keys of every fourth tile); at the end the waves extract their top m
//     with wave-wide exchanges, merge by rank, and the workgroup writes its
//     top m plus a bound of the rest to its private slot; the top-k kernel
//     merges those slots (no cross-workgroup atomics or fences, which
//     serialise on this chip).
#include "common.h"
#include "kernels.h"
#include "score_tile.h"
#include "step_prep.h"
#include "topk_common.h"

namespace csa {

namespace {

constexpr int kScoreThreads = 256;  // four waves; one workgroup per CU in the grid (index_score_bf16_wgs)
constexpr int kWavesPerWg = kScoreThreads / kWave;
static_assert(kWavesPerWg == kScoreWavesPerWg, "waves per workgroup as the host assumes");
constexpr int kTileKeys = 16;
constexpr int kHeads = 64;
constexpr int kDi = 128;
constexpr int kSteps = kDi / 32;   // k-steps of the 16x16x32 MFMA
constexpr int kMTiles = kHeads / 16;
constexpr int kRing = 4;           // key tiles in flight per wave
constexpr int kQPitch = kDi + 8;   // LDS row pitch of the staged query (bank spread)
constexpr int kMaxTilesPerWave = 32;  // with candidates: at most 8 keys per lane list
constexpr int kLaneTop = 4;           // composites a lane keeps
static_assert(kRing == 4, "ring slot i feeds the list of lane group i");

static_assert(kHeads * kQPitch * sizeof(uint16_t) >= kPrepMaxD * sizeof(float), "prep roles reuse the query LDS");

// Score of one key held in LDS (as floats) for query row (b, tt): each run
// of kDi / kPer lanes takes one head (kPer elements of the key each).
// Returns the score in every thread.  red: kWavesPerWg floats of LDS.
__device__ inline float score_one_key(const ScoreArgs& a, int b, int tt, const float* key, float* red) {
    constexpr int kPer = kDi * kHeads / kScoreThreads;  // key elements per thread
    static_assert(kPer % 8 == 0 && kDi / kPer <= 8, "whole 16-byte query pieces, at most 8 lanes per head");
    const int h = threadIdx.x / (kDi / kPer);
    const int part = threadIdx.x % (kDi / kPer);
    const uint16_t* qh = static_cast<const uint16_t*>(a.q) + b * a.q_stride_b +
                         (static_cast<long long>(tt) * kHeads + h) * kDi + kPer * part;
    float dot = 0.f;
#pragma unroll
    for (int u = 0; u < kPer / 8; ++u) {
        const uint4 v = *reinterpret_cast<const uint4*>(qh + 8 * u);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            dot += bf16_to_f32(static_cast<uint16_t>(w4[e] & 0xffffu)) * key[kPer * part + 8 * u + 2 * e];
            dot += bf16_to_f32(static_cast<uint16_t>(w4[e] >> 16)) * key[kPer * part + 8 * u + 2 * e + 1];
        }
    }
    if (kDi / kPer > 1) dot += xor_lanes_f32<1>(dot);
    if (kDi / kPer > 2) dot += xor_lanes_f32<2>(dot);
    if (kDi / kPer > 4) dot += xor_lanes_f32<4>(dot);
    const float wh = a.w[b * a.w_stride_b + static_cast<long long>(tt) * kHeads + h];
    float sc = part == 0 ? wh * fmaxf(dot, 0.f) : 0.f;
    sc = wave_sum(sc);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = sc;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kWavesPerWg; ++w) tot += red[w];
    return tot;
}

template <bool kCands>
__global__ __launch_bounds__(kScoreThreads, 2) void k_index_score_bf16(ScoreArgs a, int tiles_per_row, PrepArgs p,
                                                                       int prep_wgs) {
    __shared__ __attribute__((aligned(16))) uint16_t qs[kHeads * kQPitch];
    __shared__ __attribute__((aligned(16))) float ws[kHeads];
    __shared__ CandSmem cs;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int row = blockIdx.y;
    const int b = row / a.t;
    const int tt = row - b * a.t;
    // keys already in the cache (with device counters: as the step starts)
    const int n_keys = a.dev ? dev_load(a.dev, p.swa_w > 0 ? p.swa_w : 1, a.n).n_comp : a.n;

    // 0. the decode step's small jobs (one query row per sequence), and the
    //    new key of a completed block: compressed, scored, given its own slot
    if (static_cast<int>(blockIdx.x) < prep_wgs) {
        float* ybuf = reinterpret_cast<float*>(qs);
        step_prep_role(p, blockIdx.x, b, ybuf, ws, ybuf);
        const bool completes = p.dev ? dev_completes(dev_load(p.dev, p.swa_w, p.max_comp), p.m, p.max_comp)
                                     : p.completes != 0;
        if (blockIdx.x == 2 && !completes && kCands && p.dev && threadIdx.x <= a.cands.m)  // an empty last slot
            a.cands.lists[(static_cast<long long>(row) * a.cands.slots + a.cands.slots - 1) * (a.cands.m + 1) +
                          threadIdx.x] = 0ull;
        if (blockIdx.x == 2 && completes) {
            float sc = score_one_key(a, b, tt, ybuf, ws + 8);
            const int key = n_keys;
            if (a.q_pos && static_cast<long long>(a.ratio) * key + a.ratio - 1 > a.q_pos[row]) sc = -INFINITY;
            if (threadIdx.x == 0) a.scores[b * a.s_stride_b + static_cast<long long>(tt) * a.ld_s + key] = sc;
            if (kCands && threadIdx.x <= a.cands.m) {
                const uint32_t kk = score_key(sc);
                u64* slot = a.cands.lists + (static_cast<long long>(row) * a.cands.slots + a.cands.slots - 1) *
                                                (a.cands.m + 1);
                slot[threadIdx.x] = (threadIdx.x == 0 && key_valid(kk, sc)) ? composite(kk, static_cast<uint32_t>(key)) : 0ull;
            }
        }
        return;
    }
    const int wg = blockIdx.x - prep_wgs;  // scan workgroup of this row
    const int scan_wgs = gridDim.x - prep_wgs;
    const int li = lane & 15;   // key column of B / head row of A within a 16-tile
    const int lg = lane >> 4;   // 8-element group of each 32-wide k-step
    const int n = n_keys;
    if (a.dev) tiles_per_row = (n + kTileKeys - 1) / kTileKeys;
    if (n <= 0) {  // nothing to scan: an empty candidate list
        if (kCands && threadIdx.x <= a.cands.m)
            a.cands.lists[(static_cast<long long>(row) * a.cands.slots + wg) * (a.cands.m + 1) + threadIdx.x] = 0ull;
        return;
    }
    const int waves_per_row = scan_wgs * kWavesPerWg;
    const int gw = wg * kWavesPerWg + wv;
    const int n_mine = gw < tiles_per_row ? (tiles_per_row - gw + waves_per_row - 1) / waves_per_row : 0;

    const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + b * a.k_stride_b + 8 * lg;
    auto load_tile = [&](int j, bf16x8* dst) {
        const int key = j < n_mine ? min((gw + j * waves_per_row) * kTileKeys + li, n - 1) : n - 1;
        const uint16_t* p = kbase + static_cast<long long>(key) * kDi;
#pragma unroll
        for (int s = 0; s < kSteps; ++s) dst[s] = *reinterpret_cast<const bf16x8*>(p + 32 * s);
    };

    // 1. query (16 KB: four 16-byte pieces per thread) and head weights first,
    //    then the first kRing key tiles, so that waiting for the query below
    //    leaves the key loads in flight
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + b * a.q_stride_b +
                           static_cast<long long>(tt) * kHeads * kDi;
    static_assert(kHeads * kDi / 8 == 4 * kScoreThreads, "four 16-byte query pieces per thread");
    auto qpiece = [&](int u) -> uint4 {
        const int c = threadIdx.x + u * kScoreThreads;
        return *reinterpret_cast<const uint4*>(qrow + (c / (kDi / 8)) * kDi + (c % (kDi / 8)) * 8);
    };
    const uint4 qv0 = qpiece(0), qv1 = qpiece(1), qv2 = qpiece(2), qv3 = qpiece(3);
    const float* wrow = a.w + b * a.w_stride_b + static_cast<long long>(tt) * kHeads;
    const float4 wv4 = *reinterpret_cast<const float4*>(wrow + 4 * (threadIdx.x & 15));
    // keep the key loads younger than the query loads (the wait below is in order)
    __builtin_amdgcn_sched_barrier(0);
    // Ring refills are unconditional so every iteration issues the same loads
    // (the wait counts stay exact); slots past this wave's last tile re-read
    // the row's last key, which stays in L2.
    bf16x8 kb[kRing][kSteps];
#pragma unroll
    for (int i = 0; i < kRing; ++i) load_tile(i, kb[i]);

    // 2. stage the query and weights through LDS into registers
    auto qstage = [&](int u, const uint4& v) {
        const int c = threadIdx.x + u * kScoreThreads;
        *reinterpret_cast<uint4*>(qs + (c / (kDi / 8)) * kQPitch + (c % (kDi / 8)) * 8) = v;
    };
    qstage(0, qv0);
    qstage(1, qv1);
    qstage(2, qv2);
    qstage(3, qv3);
    if (threadIdx.x < 16) *reinterpret_cast<float4*>(ws + 4 * threadIdx.x) = wv4;  // ws: 64 floats
    __syncthreads();
    bf16x8 qa[kMTiles][kSteps];
#pragma unroll
    for (int mt = 0; mt < kMTiles; ++mt)
#pragma unroll
        for (int s = 0; s < kSteps; ++s)
            qa[mt][s] = *reinterpret_cast<const bf16x8*>(qs + (16 * mt + li) * kQPitch + 32 * s + 8 * lg);
    float wr[kMTiles][4];
#pragma unroll
    for (int mt = 0; mt < kMTiles; ++mt) {
        const float4 v = *reinterpret_cast<const float4*>(ws + 16 * mt + 4 * lg);
        wr[mt][0] = v.x; wr[mt][1] = v.y; wr[mt][2] = v.z; wr[mt][3] = v.w;
    }

    float* srow = a.scores + b * a.s_stride_b + static_cast<long long>(tt) * a.ld_s;
    const long long pos = a.q_pos ? static_cast<long long>(a.q_pos[row]) : 0;
    u64 top[kLaneTop];
    u64 drop = 0;
#pragma unroll
    for (int i = 0; i < kLaneTop; ++i) top[i] = 0;
    // every lane holds the score of key li of each tile; the four tiles of a
    // ring cycle wait here and lane group lg inserts the one of tile lg
    u64 pend[kRing];

    // 3. stream: consume a tile, refill its ring slot kRing tiles ahead.
    //    The steady loop only refills tiles that exist; one more group may
    //    refill past the end (clamped, as in the preload); the last group
    //    refills nothing.  Every path leaves the same loads in flight, so the
    //    waits stay exact, and no useless load is left outstanding at the end.
    auto step = [&](int i, int j, bool refill) {
        f32x4 acc[kMTiles];
#pragma unroll
        for (int mt = 0; mt < kMTiles; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kSteps; ++s)
#pragma unroll
            for (int mt = 0; mt < kMTiles; ++mt)
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][s], kb[i][s], acc[mt], 0, 0, 0);
        if (refill) load_tile(j + kRing, kb[i]);
        const float part = tile_head_sum(acc, wr);
        const int key = (gw + j * waves_per_row) * kTileKeys + li;
        const bool live = j < n_mine && key < n;
        float sc = part;
        if (a.q_pos && static_cast<long long>(a.ratio) * key + a.ratio - 1 > pos) sc = -INFINITY;
        if (live && lg == 0) srow[key] = sc;
        if (kCands) {
            const uint32_t kk = score_key(sc);
            pend[i] = (live && key_valid(kk, sc)) ? composite(kk, static_cast<uint32_t>(key)) : 0ull;
            if (i == kRing - 1)
                lane_insert(top, drop, lg == 0 ? pend[0] : lg == 1 ? pend[1] : lg == 2 ? pend[2] : pend[3]);
        }
    };
    int j0 = 0;
    for (; j0 + 2 * kRing <= n_mine; j0 += kRing)
#pragma unroll
        for (int i = 0; i < kRing; ++i) step(i, j0 + i, true);
    if (j0 + kRing < n_mine) {  // wave-uniform
#pragma unroll
        for (int i = 0; i < kRing; ++i) step(i, j0 + i, true);
        j0 += kRing;
    }
#pragma unroll
    for (int i = 0; i < kRing; ++i) step(i, j0 + i, false);

    if (!kCands) return;
    // 4. this workgroup's best m and their bound to its candidate slot
    block_top_m<kWavesPerWg>(top, drop, a.cands.m, a.cands.mw,
                a.cands.lists + (static_cast<long long>(row) * a.cands.slots + wg) * (a.cands.m + 1), cs);
}

// float32 path (small correctness workloads): lane h of a wave takes indexer
// head h (h_i <= 64), so a key's 64 dot products run side by side and one
// wave-wide sum gives its score.  A workgroup stages the query (row pitch
// d_i + 1: lanes reading one column hit distinct banks), the head weights and
// its 16 keys in LDS; each wave scores 4 keys at once, reading every query
// element once for all four.
constexpr int kScoreF32Threads = 256;
constexpr int kScoreF32Keys = 16;
constexpr int kScoreF32PerWave = kScoreF32Keys / (kScoreF32Threads / kWave);

__global__ __launch_bounds__(kScoreF32Threads) void k_index_score_f32(ScoreArgs a) {
    extern __shared__ float qs[];  // [h_i][d_i + 1] query, [h_i] weights, [16][d_i] keys
    const int row = blockIdx.y;
    const int b = row / a.t;
    const int tt = row - b * a.t;
    const int di = a.d_i;
    const int qp = di + 1;
    float* ws = qs + a.h_i * qp;
    float* ks = ws + a.h_i;
    const float* qrow = static_cast<const float*>(a.q) + b * a.q_stride_b + static_cast<long long>(tt) * a.h_i * di;
    const float* wrow = a.w + b * a.w_stride_b + static_cast<long long>(tt) * a.h_i;
    for (int i = threadIdx.x; i < a.h_i * di; i += blockDim.x) qs[(i / di) * qp + i % di] = qrow[i];
    for (int i = threadIdx.x; i < a.h_i; i += blockDim.x) ws[i] = wrow[i];
    const int key0 = blockIdx.x * kScoreF32Keys;
    const float* kbase = static_cast<const float*>(a.k) + b * a.k_stride_b;
    for (int i = threadIdx.x; i < kScoreF32Keys * di; i += blockDim.x) {
        const int key = key0 + i / di;
        ks[i] = key < a.n ? kbase[static_cast<long long>(key) * di + i % di] : 0.f;
    }
    __syncthreads();
    const int lane = threadIdx.x & (kWave - 1);
    const int j0 = (threadIdx.x / kWave) * kScoreF32PerWave;  // this wave's first key of the workgroup
    const int h = lane < a.h_i ? lane : 0;
    const float* qh = qs + h * qp;
    const float* kj = ks + j0 * di;
    float dot[kScoreF32PerWave] = {};
    for (int d = 0; d < di; ++d) {
        const float qv = qh[d];
#pragma unroll
        for (int u = 0; u < kScoreF32PerWave; ++u) dot[u] = fmaf(qv, kj[u * di + d], dot[u]);
    }
    float sc[kScoreF32PerWave];
#pragma unroll
    for (int u = 0; u < kScoreF32PerWave; ++u) sc[u] = wave_sum(lane < a.h_i ? ws[h] * fmaxf(dot[u], 0.f) : 0.f);
    if (lane < kScoreF32PerWave) {
        float v = sc[0];
#pragma unroll
        for (int u = 1; u < kScoreF32PerWave; ++u) v = lane == u ? sc[u] : v;
        const int key = key0 + j0 + lane;
        if (key < a.n) {
            if (a.q_pos && static_cast<long long>(a.ratio) * key + a.ratio - 1 > a.q_pos[row]) v = -INFINITY;
            a.scores[b * a.s_stride_b + static_cast<long long>(tt) * a.ld_s + key] = v;
        }
    }
}

}  // namespace

int index_score_bf16_wgs(int rows, int n, int extra) {
    const int tiles = (n + kTileKeys - 1) / kTileKeys;
    // one workgroup per CU in all, the extra ones included: with the ring
    // of 4 tiles per wave that is 16 MB of key loads in flight at 1M
    // context, so the query every workgroup reads first is not queued behind
    // 32 MB (two per CU: scan 16.6 us, step 1010 steps/s; one: 16.1 us, 1039)
    const int target = device_cu_count();
    int wgs = (target + rows - 1) / rows - extra;
    // at least kRing tiles per wave where the row is long enough
    const int max_wgs = (tiles + kWavesPerWg * kRing - 1) / (kWavesPerWg * kRing);
    if (wgs > max_wgs) wgs = max_wgs;
    return wgs < 1 ? 1 : wgs;
}

int index_score_bf16_keys_per_wg(int rows, int n, int extra) {
    const int tiles = (n + kTileKeys - 1) / kTileKeys;
    const int waves = index_score_bf16_wgs(rows, n, extra) * kWavesPerWg;
    const int per_wave = (tiles + waves - 1) / waves;
    return per_wave <= kMaxTilesPerWave ? per_wave * kWavesPerWg * kTileKeys : -1;
}

hipError_t launch_index_score_bf16(const ScoreArgs& a, const PrepArgs* fold, hipStream_t s) {
    const int rows = a.batch * a.t;
    if (rows == 0 || (a.n == 0 && !fold)) return hipSuccess;
    const int tiles = (a.n + kTileKeys - 1) / kTileKeys;
    PrepArgs p{};
    int prep_wgs = 0;
    if (fold) {
        if (a.t != 1) return hipErrorInvalidValue;
        p = *fold;
        prep_wgs = p.completes ? 3 : 1;
    }
    const int wgs = index_score_bf16_wgs(rows, a.n, prep_wgs);
    const int new_slot = fold && p.completes ? 1 : 0;
    if (a.cands.lists && a.cands.slots == wgs + new_slot && (a.n == 0 || index_score_bf16_keys_per_wg(rows, a.n, prep_wgs) > 0))
        hipLaunchKernelGGL(k_index_score_bf16<true>, dim3(prep_wgs + wgs, rows), dim3(kScoreThreads), 0, s, a, tiles,
                           p, prep_wgs);
    else if (!a.cands.lists)
        hipLaunchKernelGGL(k_index_score_bf16<false>, dim3(prep_wgs + wgs, rows), dim3(kScoreThreads), 0, s, a, tiles,
                           p, prep_wgs);
    else
        return hipErrorInvalidValue;  // candidate slots that do not match the grid
    return hipGetLastError();
}

hipError_t launch_index_score_f32(const ScoreArgs& a, hipStream_t s) {
    if (a.n == 0) return hipSuccess;
    const int rows = a.batch * a.t;
    if (a.h_i > kWave) return hipErrorInvalidValue;
    const size_t lds =
        sizeof(float) * (static_cast<size_t>(a.h_i) * (a.d_i + 1) + a.h_i + static_cast<size_t>(kScoreF32Keys) * a.d_i);
    hipLaunchKernelGGL(k_index_score_f32, dim3((a.n + kScoreF32Keys - 1) / kScoreF32Keys, rows),
                       dim3(kScoreF32Threads), lds, s, a);
    return hipGetLastError();
}

}  // namespace csa

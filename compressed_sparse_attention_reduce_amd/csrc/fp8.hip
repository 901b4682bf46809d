// FP8 E4M3 indexer keys: per-row quantisation and the FP8 index score.
//
// The pages store the indexer keys as FP8_E4M3 in the KV cache for their
// tensor-core scoring path (page 1, single_shot_inference.py, "B2: FP8
// tensor-core scoring path").  Here a key row s holds 128 E4M3 codes and one
// float32 scale, K[s] = e4m3(codes) * scale[s]; the query is E4M3 too, with
// its per-head scale folded into the head weights by the caller (for c > 0,
// ReLU(c x) = c ReLU(x)).  E4M3 is the OCP encoding (bias 7, subnormals,
// NaN at S.1111.111, 448 max), which gfx950's FP8 MFMA decodes.
//
// k_quantize_fp8: one wave per row: scale = max|row| / 448 (1 for a zero
//   row), each element divided by it in binary32 and encoded by round to
//   nearest, ties to the even code, saturating at 448 (integer arithmetic on
//   the binary32 bits, no conversion instruction).
// k_index_score_fp8: the bf16 scan's design with half the bytes per key:
//   v_mfma_scale_f32_16x16x128_f8f6f4 (both formats E4M3, unit block scales:
//   one instruction per 16-head tile covers the whole 128-byte key, at twice
//   the rate of the 32-wide FP8 form), heads as M, 16-key tiles as N; each
//   lane loads 32 contiguous bytes of its key row and supplies the same 32
//   bytes of its query row, so the instruction pairs the same byte of query
//   and key whatever order it takes k slots in; the key's scale multiplies
//   the head sum (s > 0: sum_h w ReLU(s x) = s sum_h w ReLU(x)); a ring of 4
//   tiles per wave (half the bf16 kernel's bytes in flight, so the query
//   arrives sooner behind them).
//
// FP4 keys (the FP4 indexer cache the pages plan, page 1,
// ARCHITECTURE_AND_MEMORY_AUDIT.md, C4, paired with FP4 tensor-core
// scoring): a key row is 64 bytes of E2M1 codes (element 2 j in the low
// nibble of byte j) and four E8M0 scales, one per 32 elements.
//   k_quantize_fp4: one wave per 128 elements of a row, lane l taking
//     elements 2 l and 2 l + 1 (a 32-element block is 16 lanes): the block's
//     E8M0 exponent from its maximum by lane swaps, the elements scaled by
//     it (exact) and rounded to E2M1.
//   k_index_score_fp8<kCands, true>: the same scan with E4M3 query (unit
//     scales) against E2M1 keys (format code 4) on the same instruction, the
//     key's block scale as the per-lane B scale: for this shape an E2M1
//     operand gives lane (li, lg) elements 32 lg .. 32 lg + 31 of its key
//     (the 16 bytes at 16 lg, so block lg and its scale), while an E4M3
//     operand gives it elements 16 lg .. 16 lg + 15 in bytes 0-15 and 64 +
//     16 lg .. in bytes 16-31 (measured on gfx950), so the query operand is
//     taken in that order.  No multiply after the head sum.
#include "common.h"
#include "fp8_codec.h"
#include "kernels.h"
#include "score_tile.h"
#include "step_prep.h"
#include "topk_common.h"

namespace csa {

namespace {

constexpr int kQuantThreads = 256;
constexpr int kQuantRowsPerWg = kQuantThreads / kWave;

// w_in / w_out (a query's head weights, nullable): w_out[row] = w_in[row] *
// scale instead of scales[row] = scale (the scale folded into the weight).
__global__ __launch_bounds__(kQuantThreads) void k_quantize_fp8(const void* __restrict__ x, int x_bf16,
                                                                uint8_t* __restrict__ codes,
                                                                float* __restrict__ scales, long long rows, int d,
                                                                const float* __restrict__ w_in,
                                                                float* __restrict__ w_out) {
    const int lane = threadIdx.x & (kWave - 1);
    const long long row = static_cast<long long>(blockIdx.x) * kQuantRowsPerWg + threadIdx.x / kWave;
    if (row >= rows) return;  // wave-uniform
    auto get = [&](int j) -> float {
        const long long o = row * d + j;
        return x_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(x)[o]) : static_cast<const float*>(x)[o];
    };
    float amax = 0.f;
    for (int j = lane; j < d; j += kWave) amax = fmaxf(amax, fabsf(get(j)));
    amax = wave_max(amax);
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    for (int j = lane; j < d; j += kWave) codes[row * d + j] = e4m3_encode_rne(get(j) / scale);
    if (lane == 0) {
        if (w_out) w_out[row] = w_in[row] * scale;
        else scales[row] = scale;
    }
}

// FP4 E2M1 with E8M0 block scales: rows [rows][d] (d a multiple of 32) to
// packed codes [rows][d / 2] and scales [rows][d / 32], one wave per row,
// 128 elements per pass.
__global__ __launch_bounds__(kQuantThreads) void k_quantize_fp4(const void* __restrict__ x, int x_bf16,
                                                                uint8_t* __restrict__ codes,
                                                                uint8_t* __restrict__ scales, long long rows, int d) {
    const int lane = threadIdx.x & (kWave - 1);
    const long long row = static_cast<long long>(blockIdx.x) * kQuantRowsPerWg + threadIdx.x / kWave;
    if (row >= rows) return;  // wave-uniform
    auto get = [&](int j) -> float {
        const long long o = row * d + j;
        return x_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(x)[o]) : static_cast<const float*>(x)[o];
    };
    for (int base = 0; base < d; base += 2 * kWave) {
        const int j = base + 2 * lane;
        const bool live = j < d;  // whole 16-lane blocks (d is a multiple of 32)
        const float x0 = live ? get(j) : 0.f;
        const float x1 = live ? get(j + 1) : 0.f;
        float amax = fmaxf(fabsf(x0), fabsf(x1));
        amax = fmaxf(amax, xor_lanes_f32<1>(amax));
        amax = fmaxf(amax, xor_lanes_f32<2>(amax));
        amax = fmaxf(amax, xor_lanes_f32<4>(amax));
        amax = fmaxf(amax, xor_lanes_f32<8>(amax));
        const int xe = mx_block_exp(amax);
        const uint32_t c0 = e2m1_encode_rne(__builtin_ldexpf(x0, -xe));
        const uint32_t c1 = e2m1_encode_rne(__builtin_ldexpf(x1, -xe));
        if (live) {
            codes[row * (d / 2) + j / 2] = static_cast<uint8_t>(c0 | (c1 << 4));
            if ((lane & 15) == 0) scales[row * (d / 32) + j / 32] = static_cast<uint8_t>(xe + 127);
        }
    }
}

// ---- FP8 index score ------------------------------------------------------------

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTileKeys = 16;
constexpr int kHeads = 64;
constexpr int kDi = 128;            // key bytes (one per element)
constexpr int kMTiles = kHeads / 16;
// key tiles in flight per wave: 4 rather than 8, so that the query, which
// every workgroup reads first, is not queued behind 32 MB of key loads at
// 1M context (8 tiles: scan 10.6 us, decode step 1040 steps/s; 4 tiles:
// 9.4 us, 1131 steps/s; csa_queue_probe shows the shared row's arrival
// growing with the bytes in flight)
constexpr int kRing = 4;
constexpr int kQPitch = kDi + 16;   // LDS row pitch of the staged query (bytes)

constexpr int kLaneTop = 4;         // composites a lane keeps (candidate lists)
constexpr int kMaxTilesPerWave = 32;  // with candidates: at most 8 keys per lane list
static_assert(kRing % 4 == 0, "each run of four ring slots feeds the four lane groups' lists");

static_assert(kWaves == kScoreWavesPerWg, "waves per workgroup as the host assumes");

typedef int i32x8 __attribute__((ext_vector_type(8)));  // 32 E4M3 codes, one MFMA operand
constexpr int kUnitScale = 127;  // E8M0 block scale 2^(127 - 127) = 1
constexpr int kFp8WgsPerCu = 2;  // one per CU measured slower (11.3 vs 10.9 us at n = 250,000)

// Score of the new key (decoded E4M3 values key[0..128), scale key[128], in
// LDS) for query row (b, tt): four lanes per head, 32 code bytes each.
// Returns the score in every thread; red: kWaves floats of LDS.
__device__ inline float score_one_key_fp8(const Fp8ScoreArgs& a, int b, int tt, const float* key, float* red) {
    constexpr int kPer = kDi * kHeads / kThreads;  // key elements per thread
    static_assert(kDi / kPer == 4, "four lanes per head");
    const int h = threadIdx.x / (kDi / kPer);
    const int part = threadIdx.x % (kDi / kPer);
    float wh = a.w[b * a.w_stride_b + static_cast<long long>(tt) * kHeads + h];
    float dot = 0.f;
    if (a.q_raw) {
        // bfloat16 query: the head row quantised as the scan quantises it (the
        // row maximum over the head's four lanes), its scale folded into wh
        const uint16_t* qh = a.q_raw + b * a.q_raw_stride_b + (static_cast<long long>(tt) * kHeads + h) * kDi + kPer * part;
        float x[kPer];
#pragma unroll
        for (int u = 0; u < kPer / 8; ++u) {
            const uint4 v = *reinterpret_cast<const uint4*>(qh + 8 * u);
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[8 * u + 2 * e] = bf16_to_f32(static_cast<uint16_t>(w4[e] & 0xffffu));
                x[8 * u + 2 * e + 1] = bf16_to_f32(static_cast<uint16_t>(w4[e] >> 16));
            }
        }
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < kPer; ++e) amax = fmaxf(amax, fabsf(x[e]));
        amax = fmaxf(amax, xor_lanes_f32<1>(amax));
        amax = fmaxf(amax, xor_lanes_f32<2>(amax));
        const E4m3Row rs = e4m3_row(amax);
#pragma unroll
        for (int e = 0; e < kPer; e += 2) {
            const uint32_t c2 = e4m3_encode2(e4m3_quot(x[e], rs), e4m3_quot(x[e + 1], rs));
            dot += e4m3_decode(c2 & 0xffu) * key[kPer * part + e];
            dot += e4m3_decode(c2 >> 8) * key[kPer * part + e + 1];
        }
        wh = wh * rs.s;
    } else {
        const uint8_t* qh = a.q + b * a.q_stride_b + (static_cast<long long>(tt) * kHeads + h) * kDi + kPer * part;
#pragma unroll
        for (int u = 0; u < kPer / 16; ++u) {
            const uint4 v = *reinterpret_cast<const uint4*>(qh + 16 * u);
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 16; ++e)
                dot += e4m3_decode((w4[e >> 2] >> (8 * (e & 3))) & 0xffu) * key[kPer * part + 16 * u + e];
        }
    }
    dot += xor_lanes_f32<1>(dot);
    dot += xor_lanes_f32<2>(dot);
    float sc = part == 0 ? wh * fmaxf(dot * key[kDi], 0.f) : 0.f;
    sc = wave_sum(sc);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = sc;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tot += red[w];
    return tot;
}

template <bool kCands, bool kFp4>
__global__ __launch_bounds__(kThreads, 2) void k_index_score_fp8(Fp8ScoreArgs a, int tiles_per_row, PrepArgs p,
                                                                 int prep_wgs) {
    // the query staging area doubles as the LDS of the decode step's small jobs
    constexpr int kLdsFloats = kPrepMaxD + kDi + 8;
    static_assert(kHeads * kQPitch <= kLdsFloats * sizeof(float), "query fits the shared area");
    __shared__ __attribute__((aligned(16))) float lds[kLdsFloats];
    __shared__ __attribute__((aligned(16))) float ws[kHeads];
    __shared__ __attribute__((aligned(16))) float qsc[kHeads];  // a bfloat16 query's head scales
    __shared__ CandSmem cs;
    uint8_t* qs = reinterpret_cast<uint8_t*>(lds);
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int row = blockIdx.y;
    const int b = row / a.t;
    const int tt = row - b * a.t;

    // 0. the decode step's small jobs; the workgroup that quantises the new
    //    indexer key also scores it and fills its candidate slot
    if (static_cast<int>(blockIdx.x) < prep_wgs) {
        float* ybuf = lds;
        float* key = lds + kPrepMaxD;
        step_prep_role(p, blockIdx.x, b, ybuf, ws, key);
        const bool completes = p.dev ? dev_completes(dev_load(p.dev, p.swa_w, p.max_comp), p.m, p.max_comp)
                                     : p.completes != 0;
        if (blockIdx.x == 2 && !completes && kCands && p.dev && threadIdx.x <= a.cands.m)  // an empty last slot
            a.cands.lists[(static_cast<long long>(row) * a.cands.slots + a.cands.slots - 1) * (a.cands.m + 1) +
                          threadIdx.x] = 0ull;
        if (blockIdx.x == 2 && completes) {
            float sc = score_one_key_fp8(a, b, tt, key, ws + 8);
            const int kidx = p.dev ? dev_load(p.dev, p.swa_w, p.max_comp).n_comp : a.n;
            if (a.q_pos && static_cast<long long>(a.ratio) * kidx + a.ratio - 1 > a.q_pos[row]) sc = -INFINITY;
            if (threadIdx.x == 0) a.scores[b * a.s_stride_b + static_cast<long long>(tt) * a.ld_s + kidx] = sc;
            if (kCands && threadIdx.x <= a.cands.m) {
                const uint32_t kk = score_key(sc);
                unsigned long long* slot = a.cands.lists + (static_cast<long long>(row) * a.cands.slots +
                                                            a.cands.slots - 1) * (a.cands.m + 1);
                slot[threadIdx.x] =
                    (threadIdx.x == 0 && key_valid(kk, sc)) ? composite(kk, static_cast<uint32_t>(kidx)) : 0ull;
            }
        }
        return;
    }
    const int wg = blockIdx.x - prep_wgs;
    const int scan_wgs = gridDim.x - prep_wgs;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int n = a.dev ? dev_load(a.dev, p.swa_w > 0 ? p.swa_w : 1, a.n).n_comp : a.n;
    if (a.dev) tiles_per_row = (n + kTileKeys - 1) / kTileKeys;
    if (n <= 0) {  // nothing to scan: an empty candidate list
        if (kCands && threadIdx.x <= a.cands.m)
            a.cands.lists[(static_cast<long long>(row) * a.cands.slots + wg) * (a.cands.m + 1) + threadIdx.x] = 0ull;
        return;
    }
    const int waves_per_row = scan_wgs * kWaves;
    const int gw = wg * kWaves + wv;
    const int n_mine = gw < tiles_per_row ? (tiles_per_row - gw + waves_per_row - 1) / waves_per_row : 0;

    // FP8: 32 code bytes of the key and its float scale; FP4: the 16 bytes of
    // block lg and that block's E8M0 scale (as a float's bits)
    constexpr int kKeyBytes = kFp4 ? kDi / 2 : kDi;
    const uint8_t* kbase = a.k + b * a.k_stride_b + (kFp4 ? 16 : 32) * lg;
    const float* sbase = a.k_scale + b * a.ks_stride_b;
    auto load_tile = [&](int j, uint4* dst, float& ks) {
        const int key = j < n_mine ? min((gw + j * waves_per_row) * kTileKeys + li, n - 1) : n - 1;
        const uint8_t* src = kbase + static_cast<long long>(key) * kKeyBytes;
        dst[0] = *reinterpret_cast<const uint4*>(src);
        if constexpr (kFp4) {
            dst[1] = make_uint4(0, 0, 0, 0);
            ks = __uint_as_float((__float_as_uint(sbase[key]) >> (8 * lg)) & 0xffu);
        } else {
            dst[1] = *reinterpret_cast<const uint4*>(src + 16);
            ks = sbase[key];
        }
    };

    // 1. query (8 KB of codes: two 16-byte pieces per thread; or 16 KB of
    //    bfloat16: four) and head weights, then the ring
    static_assert(kHeads * kDi / 16 == 2 * kThreads, "two 16-byte query pieces per thread");
    static_assert(kHeads * kDi / 8 == 4 * kThreads, "four 16-byte bfloat16 query pieces per thread");
    const uint8_t* qrow = a.q + b * a.q_stride_b + static_cast<long long>(tt) * kHeads * kDi;
    const uint16_t* qraw = a.q_raw + b * a.q_raw_stride_b + static_cast<long long>(tt) * kHeads * kDi;
    uint4 qv[4];
    if (a.q_raw) {
#pragma unroll
        for (int u = 0; u < 4; ++u) qv[u] = *reinterpret_cast<const uint4*>(qraw + 8 * (threadIdx.x + u * kThreads));
    } else {
        qv[0] = *reinterpret_cast<const uint4*>(qrow + 16 * threadIdx.x);
        qv[1] = *reinterpret_cast<const uint4*>(qrow + 16 * (threadIdx.x + kThreads));
    }
    const float* wrow = a.w + b * a.w_stride_b + static_cast<long long>(tt) * kHeads;
    const float4 wv4 = *reinterpret_cast<const float4*>(wrow + 4 * (threadIdx.x & 15));
    __builtin_amdgcn_sched_barrier(0);
    uint4 kb[kRing][2];
    float ksc[kRing];
#pragma unroll
    for (int i = 0; i < kRing; ++i) load_tile(i, kb[i], ksc[i]);

    // 2. stage the query and weights through LDS into registers; a bfloat16
    //    query is quantised on the way, one head row per 16 lanes (each lane
    //    8 elements): the row maximum by lane swaps, then csa_quantize_fp8's
    //    rule, and the row's scale folded into its head weight
    if (a.q_raw) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = threadIdx.x + u * kThreads;  // head c / 16, elements 8 (c % 16) ..
            const uint32_t w4[4] = {qv[u].x, qv[u].y, qv[u].z, qv[u].w};
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[2 * e] = bf16_to_f32(static_cast<uint16_t>(w4[e] & 0xffffu));
                x[2 * e + 1] = bf16_to_f32(static_cast<uint16_t>(w4[e] >> 16));
            }
            float amax = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
            amax = fmaxf(amax, xor_lanes_f32<1>(amax));
            amax = fmaxf(amax, xor_lanes_f32<2>(amax));
            amax = fmaxf(amax, xor_lanes_f32<4>(amax));
            amax = fmaxf(amax, xor_lanes_f32<8>(amax));
            const E4m3Row rs = e4m3_row(amax);
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = e4m3_quot(x[e], rs);
            const uint32_t lo = e4m3_encode2(y[0], y[1]) | (e4m3_encode2(y[2], y[3]) << 16);
            const uint32_t hi = e4m3_encode2(y[4], y[5]) | (e4m3_encode2(y[6], y[7]) << 16);
            *reinterpret_cast<uint2*>(qs + (c / 16) * kQPitch + (c % 16) * 8) = make_uint2(lo, hi);
            if ((c & 15) == 0) qsc[c / 16] = rs.s;
        }
    } else {
        auto qstage = [&](int c, const uint4& v) {
            *reinterpret_cast<uint4*>(qs + (c / (kDi / 16)) * kQPitch + (c % (kDi / 16)) * 16) = v;
        };
        qstage(threadIdx.x, qv[0]);
        qstage(threadIdx.x + kThreads, qv[1]);
    }
    if (threadIdx.x < 16) *reinterpret_cast<float4*>(ws + 4 * threadIdx.x) = wv4;
    __syncthreads();
    i32x8 qa[kMTiles];
#pragma unroll
    for (int mt = 0; mt < kMTiles; ++mt) {
        // against E4M3 keys the same 32 bytes as the key's; against E2M1 keys
        // the bytes of elements 16 lg .. and 64 + 16 lg .. (the instruction's
        // E4M3 operand order for this shape)
        const uint8_t* qp = qs + (16 * mt + li) * kQPitch + (kFp4 ? 16 : 32) * lg;
        const uint4 lo = *reinterpret_cast<const uint4*>(qp);
        const uint4 hi = *reinterpret_cast<const uint4*>(qp + (kFp4 ? 64 : 16));
        qa[mt] = i32x8{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
                       static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
    }
    float wr[kMTiles][4];
#pragma unroll
    for (int mt = 0; mt < kMTiles; ++mt) {
        const float4 v = *reinterpret_cast<const float4*>(ws + 16 * mt + 4 * lg);
        wr[mt][0] = v.x; wr[mt][1] = v.y; wr[mt][2] = v.z; wr[mt][3] = v.w;
        if (a.q_raw) {
            const float4 sc4 = *reinterpret_cast<const float4*>(qsc + 16 * mt + 4 * lg);
            wr[mt][0] *= sc4.x; wr[mt][1] *= sc4.y; wr[mt][2] *= sc4.z; wr[mt][3] *= sc4.w;
        }
    }

    float* srow = a.scores + b * a.s_stride_b + static_cast<long long>(tt) * a.ld_s;
    const long long pos = a.q_pos ? static_cast<long long>(a.q_pos[row]) : 0;
    u64 top[kLaneTop];
    u64 drop = 0;
#pragma unroll
    for (int i = 0; i < kLaneTop; ++i) top[i] = 0;
    // every lane holds the score of key li of each tile; each run of four
    // tiles waits here and lane group lg inserts the one of tile lg
    u64 pend[4];

    // 3. stream (the same ring discipline as the bf16 scan)
    auto step = [&](int i, int j, bool refill) {
        f32x4 acc[kMTiles];
#pragma unroll
        for (int mt = 0; mt < kMTiles; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const i32x8 kv = {static_cast<int>(kb[i][0].x), static_cast<int>(kb[i][0].y), static_cast<int>(kb[i][0].z),
                          static_cast<int>(kb[i][0].w), static_cast<int>(kb[i][1].x), static_cast<int>(kb[i][1].y),
                          static_cast<int>(kb[i][1].z), static_cast<int>(kb[i][1].w)};
        const float ks = ksc[i];
#pragma unroll
        for (int mt = 0; mt < kMTiles; ++mt) {
            if constexpr (kFp4)  // B: E2M1 (format 4) with the key block's E8M0 scale
                acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    qa[mt], kv, acc[mt], 0, 4, 0, kUnitScale, 0, static_cast<int>(__float_as_uint(ks)));
            else
                acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[mt], kv, acc[mt], 0, 0, 0, kUnitScale,
                                                                           0, kUnitScale);
        }
        if (refill) load_tile(j + kRing, kb[i], ksc[i]);
        // accumulator register r of M tile mt <-> head 16*mt + 4*lg + r, key li;
        // an E4M3 key's scale applied once after the head sum (ks > 0)
        const float part = kFp4 ? tile_head_sum(acc, wr) : tile_head_sum(acc, wr) * ks;
        const int key = (gw + j * waves_per_row) * kTileKeys + li;
        const bool live = j < n_mine && key < n;
        float sc = part;
        if (a.q_pos && static_cast<long long>(a.ratio) * key + a.ratio - 1 > pos) sc = -INFINITY;
        if (live && lg == 0) srow[key] = sc;
        if (kCands) {
            const uint32_t kk = score_key(sc);
            pend[i & 3] = (live && key_valid(kk, sc)) ? composite(kk, static_cast<uint32_t>(key)) : 0ull;
            if ((i & 3) == 3)
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
    block_top_m<kWaves>(top, drop, a.cands.m, a.cands.mw,
                a.cands.lists + (static_cast<long long>(row) * a.cands.slots + wg) * (a.cands.m + 1), cs);
}

}  // namespace

hipError_t launch_quantize_fp4(const void* x, bool x_bf16, uint8_t* codes, uint8_t* scales, long long rows, int d,
                               hipStream_t s) {
    if (rows == 0) return hipSuccess;
    if (d < 32 || d % 32 != 0) return hipErrorInvalidValue;
    const long long wgs = (rows + kQuantRowsPerWg - 1) / kQuantRowsPerWg;
    hipLaunchKernelGGL(k_quantize_fp4, dim3(static_cast<unsigned>(wgs)), dim3(kQuantThreads), 0, s, x,
                       x_bf16 ? 1 : 0, codes, scales, rows, d);
    return hipGetLastError();
}

hipError_t launch_quantize_fp8(const void* x, bool x_bf16, uint8_t* codes, float* scales, long long rows, int d,
                               hipStream_t s, const float* w_in, float* w_out) {
    if (rows == 0) return hipSuccess;
    const long long wgs = (rows + kQuantRowsPerWg - 1) / kQuantRowsPerWg;
    hipLaunchKernelGGL(k_quantize_fp8, dim3(static_cast<unsigned>(wgs)), dim3(kQuantThreads), 0, s, x,
                       x_bf16 ? 1 : 0, codes, scales, rows, d, w_in, w_out);
    return hipGetLastError();
}

int index_score_fp8_wgs(int rows, int n, int extra) {
    const int tiles = (n + kTileKeys - 1) / kTileKeys;
    int wgs = (kFp8WgsPerCu * device_cu_count() + rows - 1) / rows - extra;
    const int max_wgs = (tiles + kWaves * 4 - 1) / (kWaves * 4);  // at least 4 tiles per wave
    wgs = wgs > max_wgs ? max_wgs : wgs;
    return wgs < 1 ? 1 : wgs;
}

int index_score_fp8_keys_per_wg(int rows, int n, int extra) {
    const int tiles = (n + kTileKeys - 1) / kTileKeys;
    const int waves = index_score_fp8_wgs(rows, n, extra) * kWaves;
    const int per_wave = (tiles + waves - 1) / waves;
    return per_wave <= kMaxTilesPerWave ? per_wave * kWaves * kTileKeys : -1;
}

hipError_t launch_index_score_fp8(const Fp8ScoreArgs& a, const PrepArgs* fold, hipStream_t s) {
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
    const int wgs = index_score_fp8_wgs(rows, a.n, prep_wgs);
    const int new_slot = fold && p.completes ? 1 : 0;
    const bool lists = a.cands.lists != nullptr;
    if (lists && !(a.cands.slots == wgs + new_slot && (a.n == 0 || index_score_fp8_keys_per_wg(rows, a.n, prep_wgs) > 0)))
        return hipErrorInvalidValue;  // candidate slots that do not match the grid
    const dim3 grid(prep_wgs + wgs, rows);
    if (a.k_fp4) {
        if (lists) hipLaunchKernelGGL((k_index_score_fp8<true, true>), grid, dim3(kThreads), 0, s, a, tiles, p, prep_wgs);
        else hipLaunchKernelGGL((k_index_score_fp8<false, true>), grid, dim3(kThreads), 0, s, a, tiles, p, prep_wgs);
    } else {
        if (lists) hipLaunchKernelGGL((k_index_score_fp8<true, false>), grid, dim3(kThreads), 0, s, a, tiles, p, prep_wgs);
        else hipLaunchKernelGGL((k_index_score_fp8<false, false>), grid, dim3(kThreads), 0, s, a, tiles, p, prep_wgs);
    }
    return hipGetLastError();
}

}  // namespace csa

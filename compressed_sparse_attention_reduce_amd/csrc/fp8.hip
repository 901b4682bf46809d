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
//   v_mfma_f32_16x16x32_fp8_fp8, heads as M, 16-key tiles as N; each lane
//   loads 32 contiguous bytes of its key row (the MFMA's k slots are
//   permuted identically for the query and the keys: slot 8g + e of k-step s
//   is byte 32g + 8s + e), plus the key's scale; a ring of 8 tiles per wave
//   keeps as many bytes in flight as the bf16 kernel's 4.
#include "common.h"
#include "kernels.h"

namespace csa {

namespace {

__device__ inline uint8_t e4m3_encode_rne(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a >= 0x43e00000u) return static_cast<uint8_t>(sign | 0x7eu);  // |y| >= 448: saturate
    const int e = static_cast<int>(a >> 23) - 127;
    if (e >= -6) {  // normal E4M3
        const uint32_t mant = a & 0x7fffffu;
        uint32_t m3 = mant >> 20;
        const uint32_t rem = mant & 0xfffffu;
        if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ++m3;
        uint32_t ee = static_cast<uint32_t>(e + 7);
        if (m3 == 8u) {
            m3 = 0;
            ++ee;
        }
        return static_cast<uint8_t>(sign | (ee << 3) | m3);
    }
    // subnormal E4M3: m * 2^-9, m = round(|y| * 2^9) in 0..8
    const int sh = 14 - e;  // |y| * 2^9 = (1.mant * 2^23) >> sh
    if (sh >= 25) return static_cast<uint8_t>(sign);  // below half the smallest subnormal
    const uint32_t M = (a & 0x7fffffu) | 0x800000u;
    uint32_t m = M >> sh;
    const uint32_t rem = M & ((1u << sh) - 1u);
    const uint32_t half = 1u << (sh - 1);
    if (rem > half || (rem == half && (m & 1u))) ++m;
    return static_cast<uint8_t>(sign | m);
}

constexpr int kQuantThreads = 256;
constexpr int kQuantRowsPerWg = kQuantThreads / kWave;

__global__ __launch_bounds__(kQuantThreads) void k_quantize_fp8(const void* __restrict__ x, int x_bf16,
                                                                uint8_t* __restrict__ codes,
                                                                float* __restrict__ scales, long long rows, int d) {
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
    if (lane == 0) scales[row] = scale;
}

// ---- FP8 index score ------------------------------------------------------------

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTileKeys = 16;
constexpr int kHeads = 64;
constexpr int kDi = 128;            // key bytes (one per element)
constexpr int kSteps = kDi / 32;    // k-steps of the 16x16x32 MFMA
constexpr int kMTiles = kHeads / 16;
constexpr int kRing = 8;            // key tiles in flight per wave
constexpr int kQPitch = kDi + 16;   // LDS row pitch of the staged query (bytes)

typedef long fp8x8;  // eight E4M3 codes, one MFMA operand
constexpr int kFp8WgsPerCu = 2;  // one per CU measured slower (11.3 vs 10.9 us at n = 250,000)

__global__ __launch_bounds__(kThreads, 2) void k_index_score_fp8(Fp8ScoreArgs a, int tiles_per_row) {
    __shared__ __attribute__((aligned(16))) uint8_t qs[kHeads * kQPitch];
    __shared__ __attribute__((aligned(16))) float ws[kHeads];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int row = blockIdx.y;
    const int b = row / a.t;
    const int tt = row - b * a.t;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int n = a.n;
    const int waves_per_row = gridDim.x * kWaves;
    const int gw = blockIdx.x * kWaves + wv;
    const int n_mine = gw < tiles_per_row ? (tiles_per_row - gw + waves_per_row - 1) / waves_per_row : 0;

    const uint8_t* kbase = a.k + b * a.k_stride_b + 32 * lg;
    const float* sbase = a.k_scale + b * a.ks_stride_b;
    auto load_tile = [&](int j, uint4* dst, float& ks) {
        const int key = j < n_mine ? min((gw + j * waves_per_row) * kTileKeys + li, n - 1) : n - 1;
        const uint8_t* p = kbase + static_cast<long long>(key) * kDi;
        dst[0] = *reinterpret_cast<const uint4*>(p);
        dst[1] = *reinterpret_cast<const uint4*>(p + 16);
        ks = sbase[key];
    };

    // 1. query (8 KB: two 16-byte pieces per thread) and head weights, then the ring
    const uint8_t* qrow = a.q + b * a.q_stride_b + static_cast<long long>(tt) * kHeads * kDi;
    static_assert(kHeads * kDi / 16 == 2 * kThreads, "two 16-byte query pieces per thread");
    const uint4 qv0 = *reinterpret_cast<const uint4*>(qrow + 16 * threadIdx.x);
    const uint4 qv1 = *reinterpret_cast<const uint4*>(qrow + 16 * (threadIdx.x + kThreads));
    const float* wrow = a.w + b * a.w_stride_b + static_cast<long long>(tt) * kHeads;
    const float4 wv4 = *reinterpret_cast<const float4*>(wrow + 4 * (threadIdx.x & 15));
    __builtin_amdgcn_sched_barrier(0);
    uint4 kb[kRing][2];
    float ksc[kRing];
    if (n > 0) {
#pragma unroll
        for (int i = 0; i < kRing; ++i) load_tile(i, kb[i], ksc[i]);
    }

    // 2. stage the query and weights through LDS into registers
    auto qstage = [&](int c, const uint4& v) {
        *reinterpret_cast<uint4*>(qs + (c / (kDi / 16)) * kQPitch + (c % (kDi / 16)) * 16) = v;
    };
    qstage(threadIdx.x, qv0);
    qstage(threadIdx.x + kThreads, qv1);
    if (threadIdx.x < 16) *reinterpret_cast<float4*>(ws + 4 * threadIdx.x) = wv4;
    __syncthreads();
    if (n <= 0) return;
    fp8x8 qa[kMTiles][kSteps];
#pragma unroll
    for (int mt = 0; mt < kMTiles; ++mt)
#pragma unroll
        for (int s = 0; s < kSteps; ++s)
            qa[mt][s] = *reinterpret_cast<const fp8x8*>(qs + (16 * mt + li) * kQPitch + 32 * lg + 8 * s);
    float wr[kMTiles][4];
#pragma unroll
    for (int mt = 0; mt < kMTiles; ++mt) {
        const float4 v = *reinterpret_cast<const float4*>(ws + 16 * mt + 4 * lg);
        wr[mt][0] = v.x; wr[mt][1] = v.y; wr[mt][2] = v.z; wr[mt][3] = v.w;
    }

    float* srow = a.scores + b * a.s_stride_b + static_cast<long long>(tt) * a.ld_s;
    const long long pos = a.q_pos ? static_cast<long long>(a.q_pos[row]) : 0;

    // 3. stream (the same ring discipline as the bf16 scan)
    auto step = [&](int i, int j, bool refill) {
        f32x4 acc[kMTiles];
#pragma unroll
        for (int mt = 0; mt < kMTiles; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        fp8x8 kv[kSteps];
        __builtin_memcpy(kv, kb[i], sizeof(kv));
#pragma unroll
        for (int s = 0; s < kSteps; ++s)
#pragma unroll
            for (int mt = 0; mt < kMTiles; ++mt)
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(qa[mt][s], kv[s], acc[mt], 0, 0, 0);
        const float ks = ksc[i];
        if (refill) load_tile(j + kRing, kb[i], ksc[i]);
        // accumulator register r of M tile mt <-> head 16*mt + 4*lg + r, key li
        float part = 0.f;
#pragma unroll
        for (int mt = 0; mt < kMTiles; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) part += wr[mt][r] * fmaxf(acc[mt][r] * ks, 0.f);
        part += xor_lanes_f32<16>(part);
        part += xor_lanes_f32<32>(part);
        const int key = (gw + j * waves_per_row) * kTileKeys + li;
        float sc = part;
        if (a.q_pos && static_cast<long long>(a.ratio) * key + a.ratio - 1 > pos) sc = -INFINITY;
        if (j < n_mine && key < n && lg == 0) srow[key] = sc;
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
}

}  // namespace

hipError_t launch_quantize_fp8(const void* x, bool x_bf16, uint8_t* codes, float* scales, long long rows, int d,
                               hipStream_t s) {
    if (rows == 0) return hipSuccess;
    const long long wgs = (rows + kQuantRowsPerWg - 1) / kQuantRowsPerWg;
    hipLaunchKernelGGL(k_quantize_fp8, dim3(static_cast<unsigned>(wgs)), dim3(kQuantThreads), 0, s, x,
                       x_bf16 ? 1 : 0, codes, scales, rows, d);
    return hipGetLastError();
}

hipError_t launch_index_score_fp8(const Fp8ScoreArgs& a, hipStream_t s) {
    const int rows = a.batch * a.t;
    if (rows == 0 || a.n == 0) return hipSuccess;
    const int tiles = (a.n + kTileKeys - 1) / kTileKeys;
    int wgs = (kFp8WgsPerCu * device_cu_count() + rows - 1) / rows;
    const int max_wgs = (tiles + kWaves * 4 - 1) / (kWaves * 4);  // at least 4 tiles per wave
    wgs = wgs > max_wgs ? max_wgs : wgs;
    wgs = wgs < 1 ? 1 : wgs;
    hipLaunchKernelGGL(k_index_score_fp8, dim3(wgs, rows), dim3(kThreads), 0, s, a, tiles);
    return hipGetLastError();
}

}  // namespace csa

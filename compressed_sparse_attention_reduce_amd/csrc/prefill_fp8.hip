// The multi-query index score over E4M3 keys: the FP8 variant of the
// prefill chunk's scoring contraction.
//
// Page 1, ARCHITECTURE_AND_MEMORY_AUDIT.md, finding F3 (paper section 2.3.1,
// eq. 16) for the score; page 1, single_shot_inference.py, comment "B2: FP8
// tensor-core scoring path" (indexer keys stored as FP8_E4M3); the causal
// block mask of archived_plans/NEXT_STEPS.md, Issue 2.  Key s decodes to
// e4m3(code) * k_scale[s] (one float32 scale per row); the query is E4M3 with
// its per-head scale folded into w by the caller.
//
// k_index_score_mq_fp8 has the structure of the bf16 multi-query scan (eight
// waves, two query rows per wave held as A operands, 16-key tiles staged
// through LDS in groups of eight with one barrier per group, the next group
// prefetched into registers) with two changes.  The product is gfx950's
// v_mfma_scale_f32_16x16x128_f8f6f4 with both formats E4M3 and unit block
// scales: one instruction covers the whole 128-wide key of a 16-head tile, at
// twice the bf16 MFMA's rate.  Each lane supplies 32 consecutive bytes of its
// query row (A) and of its key (B) at the same offset, so whatever order the
// instruction pairs k slots in, it pairs the same byte of query and key.  And
// the key scale is applied once per key after the head sum: for s > 0,
// sum_h w[h] ReLU(s x_h) = s sum_h w[h] ReLU(x_h).
//
// kFp4: E2M1 keys with one E8M0 scale per 32 elements (the FP4 indexer cache
// of page 1, ARCHITECTURE_AND_MEMORY_AUDIT.md, C4): 64-byte key rows, four
// scale bytes per key in one 32-bit word.  The same instruction with the B
// operand as format 4 (E2M1), each lane's 16 bytes block lg of its key and
// that block's scale as its B scale; the E4M3 query operand is taken in the
// order the instruction reads it beside an E2M1 operand (bytes 0-15: k 16 lg
// .. 16 lg + 15, bytes 16-31: k 64 + 16 lg ..), and the block scales apply
// inside the instruction, so nothing multiplies after the head sum.
#include "common.h"
#include "kernels.h"
#include "prefill.h"
#include "score_tile.h"

namespace csa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kF8Heads = 64;
constexpr int kF8Di = 128;           // bytes of a key or a query head row
constexpr int kF8Tok = 2;            // query rows per wave
constexpr int kF8Waves = 8;
constexpr int kF8Threads = kF8Waves * kWave;
constexpr int kF8RowsWg = kF8Waves * kF8Tok;
constexpr int kF8Group = 8;          // 16-key tiles per LDS group
constexpr int kF8GroupKeys = 16 * kF8Group;
// key row bytes, LDS pitch (16 bytes over, so the 16 rows of a B operand
// spread over the banks), group slot and 16-byte pieces of a group per thread
template <bool kFp4> struct MqKeys {
    static constexpr int kBytes = kFp4 ? kF8Di / 2 : kF8Di;
    static constexpr int kPitch = kBytes + 16;
    static constexpr int kSlot = kF8GroupKeys * kPitch;
    static constexpr int kPieces = kF8GroupKeys * kBytes / 16 / kF8Threads;
    static constexpr int kPerKey = kBytes / 16;  // pieces of one key
};
constexpr int kF8UnitScale = 127;    // E8M0 block scale 2^(127 - 127) = 1
constexpr int kF8VmcntZero = 0x0f70; // s_waitcnt immediate: vmcnt(0), the other counters left free
static_assert(MqKeys<false>::kPieces == 2 && MqKeys<true>::kPieces == 1, "whole 16-byte pieces per thread");
static_assert(kF8GroupKeys <= kF8Threads, "one thread per key scale of a group");

struct MqFp8Args {
    const uint8_t* q;     // [B][t][64][128] E4M3
    const float* w;       // [B][t][64], query scales folded in
    const uint8_t* k;     // [B][n][128] E4M3 (E2M1: [B][n][64] packed)
    const float* k_scale; // [B][n] (E2M1: four E8M0 bytes per key, one 32-bit word)
    float* scores;        // [B][t][ld]
    int t, n;
    long long ld;
    const int* q_pos;     // [B][t] positions, or nullptr: pos0 + row (pos0 < 0: no mask)
    long long pos0;
    int ratio;
    int keys_per_wg;
    long long q_stride_b, w_stride_b, k_stride_b, ks_stride_b, s_stride_b;
};

__device__ __forceinline__ i32x8 load32(const uint8_t* p) {
    const uint4 lo = *reinterpret_cast<const uint4*>(p);
    const uint4 hi = *reinterpret_cast<const uint4*>(p + 16);
    return i32x8{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
                 static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
}

template <bool kFp4>
__global__ __launch_bounds__(kF8Threads, 1) void k_index_score_mq_fp8(MqFp8Args a) {
    using K = MqKeys<kFp4>;
    __shared__ __attribute__((aligned(16))) uint8_t keys[2 * K::kSlot];
    __shared__ float kscale[2][kF8GroupKeys];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int b = blockIdx.z;
    const int row0 = blockIdx.y * kF8RowsWg + kF8Tok * wv;  // may be >= t: such waves only load and wait
    const int k0 = blockIdx.x * a.keys_per_wg;
    const int k1 = min(a.n, k0 + a.keys_per_wg);
    if (k0 >= k1) return;  // whole workgroup
    const int n_tiles = (k1 - k0 + 15) / 16;
    const int n_groups = (n_tiles + kF8Group - 1) / kF8Group;
    int rows[kF8Tok];  // rows past the end repeat the last one; nothing of them is stored
    int vis[kF8Tok];   // keys visible to the row: key < vis (causal mask)
    const bool masked = a.q_pos || a.pos0 >= 0;
#pragma unroll
    for (int u = 0; u < kF8Tok; ++u) {
        rows[u] = min(row0 + u, a.t - 1);
        const long long p = a.q_pos ? static_cast<long long>(a.q_pos[static_cast<long long>(b) * a.t + rows[u]])
                                    : a.pos0 + rows[u];
        // block s is visible iff ratio*s + ratio - 1 <= p
        const long long v = p >= a.ratio - 1 ? (p - (a.ratio - 1)) / a.ratio + 1 : 0;
        vis[u] = !masked ? a.n : static_cast<int>(v < a.n ? v : a.n);
    }
    // lanes with (lane & 16) == 0 store row 0's score, the others row 1's
    const int odd = (lane >> 4) & 1;
    float* my_row = a.scores + b * a.s_stride_b + static_cast<long long>(rows[odd]) * a.ld;
    const int my_vis = vis[odd];

    // loader: piece p of a group is bytes 16 (p % kPerKey) .. of its key
    // p / kPerKey (a group's 128 keys are contiguous); tiles past the last one
    // repeat it and keys past the range repeat its last key, so every group
    // issues the same loads.
    const uint8_t* kb = a.k + b * a.k_stride_b;
    const float* sb = a.k_scale + b * a.ks_stride_b;
    auto group_key = [&](int g, int kig) {
        const int j = min(g * kF8Group + kig / 16, n_tiles - 1);
        return min(k0 + 16 * j + (kig & 15), k1 - 1);
    };
    auto gload = [&](int g, uint4 (&pc)[K::kPieces], float& sc) {
#pragma unroll
        for (int u = 0; u < K::kPieces; ++u) {
            const int p = threadIdx.x + u * kF8Threads;
            pc[u] = *reinterpret_cast<const uint4*>(kb + static_cast<long long>(group_key(g, p / K::kPerKey)) *
                                                             K::kBytes +
                                                    16 * (p % K::kPerKey));
        }
        sc = sb[group_key(g, threadIdx.x < kF8GroupKeys ? threadIdx.x : 0)];
    };
    auto lstore = [&](int slot, const uint4 (&pc)[K::kPieces], float sc) {
#pragma unroll
        for (int u = 0; u < K::kPieces; ++u) {
            const int p = threadIdx.x + u * kF8Threads;
            *reinterpret_cast<uint4*>(keys + slot * K::kSlot + (p / K::kPerKey) * K::kPitch + 16 * (p % K::kPerKey)) =
                pc[u];
        }
        if (threadIdx.x < kF8GroupKeys) kscale[slot][threadIdx.x] = sc;
    };

    uint4 pre[K::kPieces];
    float pre_s;
    gload(0, pre, pre_s);
    lstore(0, pre, pre_s);
    gload(1, pre, pre_s);
    i32x8 qa[kF8Tok][4];
    float wr[kF8Tok][4][4];
#pragma unroll
    for (int u = 0; u < kF8Tok; ++u) {
        const uint8_t* qr = a.q + b * a.q_stride_b + static_cast<long long>(rows[u]) * kF8Heads * kF8Di;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const uint8_t* qp = qr + (16 * mt + li) * kF8Di;
            if constexpr (kFp4) {
                const uint4 lo = *reinterpret_cast<const uint4*>(qp + 16 * lg);
                const uint4 hi = *reinterpret_cast<const uint4*>(qp + 64 + 16 * lg);
                qa[u][mt] = i32x8{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z),
                                  static_cast<int>(lo.w), static_cast<int>(hi.x), static_cast<int>(hi.y),
                                  static_cast<int>(hi.z), static_cast<int>(hi.w)};
            } else {
                qa[u][mt] = load32(qp + 32 * lg);
            }
        }
        const float* wrow = a.w + b * a.w_stride_b + static_cast<long long>(rows[u]) * kF8Heads;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const float4 v = *reinterpret_cast<const float4*>(wrow + 16 * mt + 4 * lg);
            wr[u][mt][0] = v.x; wr[u][mt][1] = v.y; wr[u][mt][2] = v.z; wr[u][mt][3] = v.w;
        }
    }
    // every prologue load lands before the loop, so the waits inside it count
    // only the loop's own prefetch
    __builtin_amdgcn_s_waitcnt(kF8VmcntZero);
    __syncthreads();

    for (int g = 0; g < n_groups; ++g) {
        const int slot = g & 1;
        if (g + 1 < n_groups) {  // uniform: park group g + 1, fetch group g + 2
            lstore(slot ^ 1, pre, pre_s);
            gload(g + 2, pre, pre_s);
        }
        const uint8_t* ks = keys + slot * K::kSlot + li * K::kPitch + (kFp4 ? 16 : 32) * lg;
#pragma unroll
        for (int i = 0; i < kF8Group; ++i) {
            const int j = min(g * kF8Group + i, n_tiles - 1);
            i32x8 kv;
            if constexpr (kFp4) {
                const uint4 lo = *reinterpret_cast<const uint4*>(ks + i * 16 * K::kPitch);
                kv = i32x8{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z),
                           static_cast<int>(lo.w), 0, 0, 0, 0};
            } else {
                kv = load32(ks + i * 16 * K::kPitch);
            }
            const float scale = kscale[slot][16 * i + li];
            const int keyc = min(k0 + 16 * j + li, k1 - 1);
            f32x4 acc[2][4];
            if constexpr (kFp4) {  // B: E2M1 (format 4) with block lg's E8M0 scale
                const int sb4 = static_cast<int>((__float_as_uint(scale) >> (8 * lg)) & 0xffu);
#pragma unroll
                for (int e = 0; e < 2; ++e)
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
                        acc[e][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            qa[e][mt], kv, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, kF8UnitScale, 0, sb4);
            } else {
#pragma unroll
                for (int e = 0; e < 2; ++e)
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
                        acc[e][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            qa[e][mt], kv, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, kF8UnitScale, 0, kF8UnitScale);
            }
            const float head = tile_head_sum2(acc[0], wr[0], acc[1], wr[1]);
            const float sc = kFp4 ? head : head * scale;
            // every lane stores (lane groups repeat the value): no branch
            my_row[keyc] = keyc < my_vis ? sc : -INFINITY;
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_index_score_mq_fp8(const Fp8ScoreArgs& sa, long long pos0, hipStream_t s) {
    if (sa.t <= 0 || sa.n <= 0 || sa.batch <= 0) return hipSuccess;
    const int groups = (sa.t + kF8RowsWg - 1) / kF8RowsWg;
    // one workgroup per CU in all; each key range is a whole number of 16-key tiles
    const long long per_split = static_cast<long long>(groups) * sa.batch;
    int splits = static_cast<int>((device_cu_count() + per_split - 1) / per_split);
    if (splits < 1) splits = 1;
    int kpw = (sa.n + splits - 1) / splits;
    kpw = (kpw + 15) / 16 * 16;
    splits = (sa.n + kpw - 1) / kpw;
    MqFp8Args a{sa.q, sa.w, sa.k, sa.k_scale, sa.scores, sa.t, sa.n, sa.ld_s, sa.q_pos, pos0, sa.ratio, kpw,
                sa.q_stride_b, sa.w_stride_b, sa.k_stride_b, sa.ks_stride_b, sa.s_stride_b};
    if (sa.k_fp4)
        hipLaunchKernelGGL(k_index_score_mq_fp8<true>, dim3(splits, groups, sa.batch), dim3(kF8Threads), 0, s, a);
    else
        hipLaunchKernelGGL(k_index_score_mq_fp8<false>, dim3(splits, groups, sa.batch), dim3(kF8Threads), 0, s, a);
    return hipGetLastError();
}

}  // namespace csa

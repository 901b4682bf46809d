// Prefill-shaped CSA chunk: T query tokens at consecutive positions against
// one compressed history (its own blocks included, hidden by the causal
// mask until complete), then per-token sparse attention.
//
// Page 1, ARCHITECTURE_AND_MEMORY_AUDIT.md, finding F3 (paper section 2.3.1,
// eq. 16) for the score; page 1, archived_plans/NEXT_STEPS.md, Issue 2 for the
// causal block mask; page 2, single_shot_inference.py, eager_attention for
// the per-query composition (score -> top-k -> one softmax over the selected
// compressed rows and the sliding window, with the sink of the D5c hunk).
//
// Score (k_index_score_mq).  With many queries the score is a dense
// [T x 64] x [128 x N] contraction, so it is bound by the matrix cores, not
// by HBM: 2 x 64 x 128 FLOP per (query, key) pair.  Each wave keeps the
// 64 x 128 query of two tokens resident as A operands (4 head tiles x 4
// k-steps of v_mfma_f32_16x16x32_bf16 each) and streams 16-key tiles as B
// operands straight from memory; the eight waves of a workgroup walk the
// same key range, so the tiles come from L1/L2 after the first wave.  The
// workgroup -> XCD assignment (consecutive workgroup ids go to consecutive
// XCDs) puts every query group of one key range on the same XCD, so each key
// range is fetched from HBM once per XCD and stays in that XCD's L2.  The
// per-tile epilogue is the decode scan's (score_tile.h), so both produce the
// same bits.  Scores of up to kPrefillChunkRows queries are held in the
// workspace at a time (67 MB at N = 65536: resident in the 256 MB
// last-level cache) and selected by the top-k kernels before the next chunk.
//
// Attention (k_prefill_attn).  One workgroup per query token computes all 64
// heads, so each selected row is read once per token.  Rows arrive in
// chunks of 32 (compressed rows by index, then the window rows, oldest
// first), staged in LDS both row-major (for S^T = K Q^T) and transposed (for
// O^T = V^T P^T), so every MFMA operand is a contiguous LDS read and the
// probabilities never leave registers: the S^T accumulator layout of a lane
// (rows 4*lg + r and 16 + 4*lg + r, head li) is exactly its B operand of the
// PV product.  Online softmax across chunks; the next chunk's rows are
// loaded into registers while the current one is computed.
#include "common.h"
#include "kernels.h"
#include "mixed_kv.h"
#include "prefill.h"
#include "score_tile.h"

namespace csa {

namespace {

__host__ __device__ inline size_t pf_align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// ---------------------------------------------------------------------------
// multi-query index score
// ---------------------------------------------------------------------------

constexpr int kIdxHeads = 64;
constexpr int kIdxDi = 128;
constexpr int kIdxSteps = kIdxDi / 32;

// Shape of the multi-query scan: query rows per wave, waves per workgroup,
// key tiles per LDS group.  16 query rows per workgroup either way.
#ifndef CSA_MQ_SHAPE
#define CSA_MQ_SHAPE 2, 8, 8
#endif
template <int kTok, int kWaves, int kGroup>
struct MqShape {
    static constexpr int kThreads = kWaves * kWave;
    static constexpr int kRows = kWaves * kTok;
    static constexpr int kGroupTiles = kGroup;
};
using Mq = MqShape<CSA_MQ_SHAPE>;
constexpr int kMqRowsPerWg = Mq::kRows;
constexpr int kMqPitch = kIdxDi + 8;  // LDS key row: 272 B, so the 16 rows of a B operand spread over the banks
constexpr size_t kMqLds = sizeof(uint16_t) * 2 * Mq::kGroupTiles * 16 * kMqPitch;

struct MqArgs {
    const uint16_t* q;   // [B][t][64][128]
    const float* w;      // [B][t][64]
    const uint16_t* k;   // [B][n][128]
    float* scores;       // [B][t][ld]
    int t, n;
    long long ld;
    const int* q_pos;    // [B][t] positions, or nullptr: pos0 + row (pos0 < 0: no mask)
    long long pos0;
    int ratio;
    int keys_per_wg;
    long long q_stride_b, w_stride_b, k_stride_b, s_stride_b;
};

// Every workgroup walks its key range in groups of kGroup 16-key tiles (4 KB
// each, contiguous in memory).  Each thread owns one piece of every tile; it
// holds the next group's pieces in registers while the current group is
// computed from LDS, parks them in the other LDS slot at the start of the
// next group and meets the others at one barrier per group, so the waves of
// a SIMD drift apart within a group and one's MFMAs overlap the other's
// epilogue.  The slot written at group g was last read at group g - 1,
// before the previous barrier.
template <int kMqTok, int kMqWaves, int kGroup>
__global__ __launch_bounds__(kMqWaves * kWave, 1) void k_index_score_mq(MqArgs a) {
    constexpr int kThreads = kMqWaves * kWave;
    constexpr int kRowsWg = kMqWaves * kMqTok;
    constexpr int kPer = 16 * kIdxDi / kThreads;  // bf16 elements of a tile per thread
    constexpr int kSlot = kGroup * 16 * kMqPitch; // elements of one LDS group slot
    static_assert(kPer == 8 || kPer == 4 || kPer == 2, "one 16-, 8- or 4-byte piece per thread");
    static_assert(kMqTok % 2 == 0, "query rows go through the epilogue in pairs");
    using Piece = typename std::conditional<kPer == 8, uint4,
                                            typename std::conditional<kPer == 4, uint2, uint32_t>::type>::type;
    extern __shared__ __attribute__((aligned(16))) uint16_t mq_lds[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int b = blockIdx.z;
    const int row0 = blockIdx.y * kRowsWg + kMqTok * wv;  // may be >= t: such waves only load and wait
    const int k0 = blockIdx.x * a.keys_per_wg;
    const int k1 = min(a.n, k0 + a.keys_per_wg);
    if (k0 >= k1) return;  // whole workgroup
    const int n_tiles = (k1 - k0 + 15) / 16;
    const int n_groups = (n_tiles + kGroup - 1) / kGroup;
    int rows[kMqTok];  // rows past the end repeat the last one; nothing of them is stored
    int vis[kMqTok];   // keys visible to the row: key < vis (causal mask)
    const bool masked = a.q_pos || a.pos0 >= 0;
#pragma unroll
    for (int u = 0; u < kMqTok; ++u) {
        rows[u] = min(row0 + u, a.t - 1);
        const long long p = a.q_pos ? static_cast<long long>(a.q_pos[static_cast<long long>(b) * a.t + rows[u]])
                                    : a.pos0 + rows[u];
        // block s is visible iff ratio*s + ratio - 1 <= p
        const long long v = p >= a.ratio - 1 ? (p - (a.ratio - 1)) / a.ratio + 1 : 0;
        vis[u] = !masked ? a.n : static_cast<int>(v < a.n ? v : a.n);
    }
    const uint16_t* qb = a.q + b * a.q_stride_b;
    const float* wb = a.w + b * a.w_stride_b;
    // row pair v: lanes of rows 1 and 3 (lane & 16) store row 2v + 1, the others row 2v
    const int odd = (lane >> 4) & 1;
    float* my_row[kMqTok / 2];
    int my_vis[kMqTok / 2];
#pragma unroll
    for (int v = 0; v < kMqTok / 2; ++v) {
        my_row[v] = a.scores + b * a.s_stride_b + static_cast<long long>(rows[2 * v + odd]) * a.ld;
        my_vis[v] = odd ? vis[2 * v + 1] : vis[2 * v];
    }

    // loader: thread -> (key of the tile, element offset in the row)
    const int lk = threadIdx.x / (kIdxDi / kPer);
    const int lo = (threadIdx.x % (kIdxDi / kPer)) * kPer;
    const uint16_t* kbase = a.k + b * a.k_stride_b + lo;
    auto gload = [&](int j) -> Piece {
        const int key = min(k0 + 16 * min(j, n_tiles - 1) + lk, k1 - 1);
        return *reinterpret_cast<const Piece*>(kbase + static_cast<long long>(key) * kIdxDi);
    };
    auto lstore = [&](int slot, int i, const Piece& v) {
        *reinterpret_cast<Piece*>(mq_lds + slot * kSlot + i * 16 * kMqPitch + lk * kMqPitch + lo) = v;
    };

    Piece pre[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) pre[i] = gload(i);
#pragma unroll
    for (int i = 0; i < kGroup; ++i) lstore(0, i, pre[i]);
#pragma unroll
    for (int i = 0; i < kGroup; ++i) pre[i] = gload(kGroup + i);
    bf16x8 qa[kMqTok][4][kIdxSteps];
    float wr[kMqTok][4][4];
#pragma unroll
    for (int u = 0; u < kMqTok; ++u) {
        const uint16_t* qr = qb + static_cast<long long>(rows[u]) * kIdxHeads * kIdxDi;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int s = 0; s < kIdxSteps; ++s)
                qa[u][mt][s] = *reinterpret_cast<const bf16x8*>(qr + (16 * mt + li) * kIdxDi + 32 * s + 8 * lg);
        const float* wrow = wb + static_cast<long long>(rows[u]) * kIdxHeads;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const float4 v = *reinterpret_cast<const float4*>(wrow + 16 * mt + 4 * lg);
            wr[u][mt][0] = v.x; wr[u][mt][1] = v.y; wr[u][mt][2] = v.z; wr[u][mt][3] = v.w;
        }
    }
    // Every load so far (query, weights, the next group's pieces) lands before
    // the loop: otherwise the wait inserted for the query registers inside the
    // loop also waits, at run time, for the prefetch issued in the loop.
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
    __syncthreads();

    for (int g = 0; g < n_groups; ++g) {
        const int slot = g & 1;
        if (g + 1 < n_groups) {  // uniform: park group g + 1, fetch group g + 2
#pragma unroll
            for (int i = 0; i < kGroup; ++i) lstore(slot ^ 1, i, pre[i]);
#pragma unroll
            for (int i = 0; i < kGroup; ++i) pre[i] = gload((g + 2) * kGroup + i);
        }
        const uint16_t* ks = mq_lds + slot * kSlot + li * kMqPitch + 8 * lg;
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            // tiles past the last one repeat it (clamped loads): no branch, so
            // every group issues the same memory operations
            const int j = min(g * kGroup + i, n_tiles - 1);
            bf16x8 kb[kIdxSteps];
#pragma unroll
            for (int s = 0; s < kIdxSteps; ++s)
                kb[s] = *reinterpret_cast<const bf16x8*>(ks + i * 16 * kMqPitch + 32 * s);
            // past-the-end keys repeat the last one (same data, same value)
            const int keyc = min(k0 + 16 * j + li, k1 - 1);
            // rows in pairs: the products of both, then one epilogue that
            // leaves row 2v's score in lanes of rows 0/2, row 2v+1's in 1/3
#pragma unroll
            for (int v = 0; v < kMqTok / 2; ++v) {
                f32x4 acc[2][4];
#pragma unroll
                for (int e = 0; e < 2; ++e)
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) acc[e][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < kIdxSteps; ++s)
#pragma unroll
                    for (int e = 0; e < 2; ++e)
#pragma unroll
                        for (int mt = 0; mt < 4; ++mt)
                            acc[e][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[2 * v + e][mt][s], kb[s],
                                                                                 acc[e][mt], 0, 0, 0);
                const float sc = tile_head_sum2(acc[0], wr[2 * v], acc[1], wr[2 * v + 1]);
                // every lane stores (lane groups repeat the value): no branch
                my_row[v][keyc] = keyc < my_vis[v] ? sc : -INFINITY;
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// per-query attention over indexed rows + the sliding window
// ---------------------------------------------------------------------------

constexpr int kPaThreads = 256;          // four waves: one 16-head tile each (h <= 64)
constexpr int kPaWaves = kPaThreads / kWave;
// The softmax reference max moves only when a chunk's max exceeds it by more
// than this (natural-log units): exp(s - ref) then stays below e^8, far from
// float or bfloat16 overflow, and the output is rescaled rarely (never, for
// logits of unit scale) instead of at every chunk.
constexpr float kLazyRescale = 8.f;

// Slot swizzle of the transposed rows: columns 16 B apart (cc, cc + 1) share
// a bank offset once the column pitch is taken mod 256 B, so their row
// groups are xor-ed with cc / 2 (the 16 columns of one PV read share it).
// Two floats to packed bfloat16 (round to nearest even, the low half from a):
// one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
    const __bf16 ha = static_cast<__bf16>(a);
    const __bf16 hb = static_cast<__bf16>(b);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, ha)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hb)) << 16);
}

template <int kSlots>
__device__ __forceinline__ int pa_swz(int cc) { return (cc >> 1) & (kSlots - 1); }

template <int D>
struct PaCfg {
    static constexpr int kRows = 32;  // rows per chunk: 74 KB of LDS at D = 512, two workgroups per CU
    static constexpr int kMt = kRows / 16;                  // 16-row tiles of S^T
    static constexpr int kKrPitch = D + 8;                  // row-major rows: 16-lane reads hit distinct banks
    static constexpr int kVtPitch = kRows + 8;              // transposed rows: 80 B per column
    static constexpr int kKs = D / 32;                      // k-steps of S^T
    static constexpr int kMd = D / 16;                      // 16-column tiles of O^T
    static constexpr int kItems = (kRows / 4) * (D / 8);    // (4-row group, 16-byte column) items per chunk
    static constexpr int kIpt = (kItems + kPaThreads - 1) / kPaThreads;
    static constexpr size_t kLdsRows = sizeof(uint16_t) * (static_cast<size_t>(kRows) * kKrPitch +
                                                          static_cast<size_t>(D) * kVtPitch);
};

// Two workgroups per CU: one's loads and barriers overlap the other's
// matrix work (at D = 512 a few registers spill to scratch: measured 10%
// faster than one workgroup per CU with 64-row chunks all the same).
// kMixed (D = 512): the rows are mixed records; a NoPE item reads its 8 codes
// and the row scale and is decoded to bfloat16 before the LDS stores, a RoPE
// item is 16 bytes of the record's bf16 part, and the output's RoPE pairs are
// rotated back at the query's position.
template <int D, bool kMixed>
__global__ __launch_bounds__(kPaThreads, 2) void k_prefill_attn(PrefillAttnArgs a) {
    using C = PaCfg<D>;
    constexpr int R = C::kRows;
    extern __shared__ __attribute__((aligned(16))) uint16_t pa_lds[];
    uint16_t* kr = pa_lds;                                      // [R][D + 8]
    uint16_t* vt = kr + R * C::kKrPitch;                        // [D][R + 8]
    int* sidx = reinterpret_cast<int*>(vt + D * C::kVtPitch);   // [k]
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int tq = blockIdx.x;
    const long long p = a.pos0 + tq;
    const int wl = static_cast<int>(min(static_cast<long long>(a.window), p + 1));
    int cnt = a.count ? a.count[tq] : a.k;
    cnt = cnt < 0 ? 0 : (cnt > a.k ? a.k : cnt);
    if (a.n_comp <= 0) cnt = 0;
    const int nv = cnt + wl;
    const bool active = 16 * wv < a.h;
    // the token's first window row (element or record units)
    const long long win_row0 = static_cast<long long>(tq) + a.window - wl;
    const uint16_t* win = a.win_kv + win_row0 * D;
    const uint8_t* comp_rec = reinterpret_cast<const uint8_t*>(a.comp_kv);
    const uint8_t* win_rec = reinterpret_cast<const uint8_t*>(a.win_kv) + win_row0 * kMixRec;

    // this token's selected indices to LDS; the query tile's B operands
    const int* idx = a.idx + static_cast<long long>(tq) * a.k;
    for (int j = threadIdx.x; j < cnt; j += kPaThreads) {
        const int r = idx[j];
        sidx[j] = r < 0 ? 0 : (r >= a.n_comp ? a.n_comp - 1 : r);
    }
    bf16x8 qb[C::kKs];
    if (active) {
        const uint16_t* qh = a.q + (static_cast<long long>(tq) * a.h + 16 * wv + li) * D + 8 * lg;
#pragma unroll
        for (int ks = 0; ks < C::kKs; ++ks) qb[ks] = *reinterpret_cast<const bf16x8*>(qh + 32 * ks);
    }
    __syncthreads();

    // Items (4-row group rg, 16-byte column cc), column fastest: a wave loads
    // whole 1 KB rows (coalesced) and writes them row-major without bank
    // conflicts.  The transposed copy puts rows 4*rg .. 4*rg + 3 of column d
    // at slot rg ^ swz(d): the columns a wave writes at once land in distinct
    // banks, and the PV reads (16 columns, one slot) stay conflict-free too.
    // Rows past the valid ones repeat the token's last row: their
    // probabilities are exactly 0 and their values finite, so they add
    // nothing, and every load is unconditional.
    const uint16_t* last_row = win + static_cast<long long>(wl - 1) * D;
    const uint8_t* last_rec = win_rec + static_cast<long long>(wl - 1) * kMixRec;
    uint4 v[C::kIpt][4];
    float vsc[C::kIpt][4];  // mixed: the row scale of each item (unused otherwise)
    auto load_chunk = [&](int j0) {
#pragma unroll
        for (int u = 0; u < C::kIpt; ++u) {
            const int it = threadIdx.x + u * kPaThreads;
            const int cc = it % (D / 8);
            const int rg = min(it / (D / 8), R / 4 - 1);  // items past the end repeat the last (not stored)
#pragma unroll
            for (int u2 = 0; u2 < 4; ++u2) {
                const int j = j0 + 4 * rg + u2;
                if constexpr (kMixed) {
                    const uint8_t* src = j < cnt ? comp_rec + static_cast<long long>(sidx[j]) * kMixRec
                                                 : (j < nv ? win_rec + static_cast<long long>(j - cnt) * kMixRec
                                                           : last_rec);
                    // one 16-byte read (8 codes, or 16 bytes of the RoPE part) and the row scale, with
                    // no branch on the item kind; decoded at the LDS store
                    v[u][u2] = mixed_piece_load(mixed_piece_ptr(src, cc));
                    vsc[u][u2] = *reinterpret_cast<const float*>(src + kMixScaleOff);
                } else {
                    const uint16_t* src = j < cnt ? a.comp_kv + static_cast<long long>(sidx[j]) * D
                                                  : (j < nv ? win + static_cast<long long>(j - cnt) * D : last_row);
                    v[u][u2] = *reinterpret_cast<const uint4*>(src + 8 * cc);
                }
            }
        }
    };
    auto store_chunk = [&]() {
#pragma unroll
        for (int u = 0; u < C::kIpt; ++u) {
            const int it = threadIdx.x + u * kPaThreads;
            if (C::kItems % kPaThreads != 0 && it >= C::kItems) continue;
            const int cc = it % (D / 8);
            const int rg = it / (D / 8);
            if constexpr (kMixed) {
#pragma unroll
                for (int u2 = 0; u2 < 4; ++u2) v[u][u2] = mixed_piece_value(v[u][u2], vsc[u][u2], cc);
            }
#pragma unroll
            for (int u2 = 0; u2 < 4; ++u2)
                *reinterpret_cast<uint4*>(kr + (4 * rg + u2) * C::kKrPitch + 8 * cc) = v[u][u2];
            // column 8*cc + e gets rows 4*rg .. 4*rg + 3 (one 8-byte write),
            // element pairs gathered by byte permutes
            const uint32_t w0[4] = {v[u][0].x, v[u][0].y, v[u][0].z, v[u][0].w};
            const uint32_t w1[4] = {v[u][1].x, v[u][1].y, v[u][1].z, v[u][1].w};
            const uint32_t w2[4] = {v[u][2].x, v[u][2].y, v[u][2].z, v[u][2].w};
            const uint32_t w3[4] = {v[u][3].x, v[u][3].y, v[u][3].z, v[u][3].w};
            const int slot = rg ^ pa_swz<R / 4>(cc);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // low halves (column 8cc + 2q), then high halves (8cc + 2q + 1)
                const uint32_t lo01 = __builtin_amdgcn_perm(w1[q], w0[q], 0x05040100u);
                const uint32_t lo23 = __builtin_amdgcn_perm(w3[q], w2[q], 0x05040100u);
                const uint32_t hi01 = __builtin_amdgcn_perm(w1[q], w0[q], 0x07060302u);
                const uint32_t hi23 = __builtin_amdgcn_perm(w3[q], w2[q], 0x07060302u);
                *reinterpret_cast<uint2*>(vt + (8 * cc + 2 * q) * C::kVtPitch + 4 * slot) = make_uint2(lo01, lo23);
                *reinterpret_cast<uint2*>(vt + (8 * cc + 2 * q + 1) * C::kVtPitch + 4 * slot) = make_uint2(hi01, hi23);
            }
        }
    };

    f32x4 o[C::kMd];
#pragma unroll
    for (int md = 0; md < C::kMd; ++md) o[md] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY, l_run = 0.f;
    const int n_chunks = (nv + R - 1) / R;
    load_chunk(0);
    for (int c = 0; c < n_chunks; ++c) {
        store_chunk();
        __syncthreads();
        if (c + 1 < n_chunks) load_chunk(R * (c + 1));
        if (active) {
            // S^T = K Q^T: lane holds rows 16*mt + 4*lg + r, head li
            f32x4 st[C::kMt];
#pragma unroll
            for (int mt = 0; mt < C::kMt; ++mt) st[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < C::kKs; ++ks)
#pragma unroll
                for (int mt = 0; mt < C::kMt; ++mt) {
                    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kr + (16 * mt + li) * C::kKrPitch + 32 * ks + 8 * lg);
                    st[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[ks], st[mt], 0, 0, 0);
                }
            const int j0 = R * c;
            float sv[4 * C::kMt];
#pragma unroll
            for (int mt = 0; mt < C::kMt; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = j0 + 16 * mt + 4 * lg + r;
                    sv[4 * mt + r] = j < nv ? st[mt][r] * a.scale : -INFINITY;
                }
            float cm = sv[0];
#pragma unroll
            for (int e = 1; e < 4 * C::kMt; ++e) cm = fmaxf(cm, sv[e]);
            cm = fmaxf(cm, xor_lanes_f32<16>(cm));
            cm = fmaxf(cm, xor_lanes_f32<32>(cm));
            // every chunk holds a valid row: cm is finite
            if (__builtin_amdgcn_ballot_w64(cm > m_ref + kLazyRescale)) {  // rare: move the reference
                const float m_new = fmaxf(m_ref, cm);
                const float alpha = expf(m_ref - m_new);  // 0 on the first chunk
                l_run *= alpha;
#pragma unroll
                for (int md = 0; md < C::kMd; ++md) o[md] *= alpha;
                m_ref = m_new;
            }
            uint32_t pb[2 * C::kMt];  // probabilities, bf16 pairs
            float ls = 0.f;
#pragma unroll
            for (int e = 0; e < 2 * C::kMt; ++e) {
                pb[e] = bf16x2_rne(expf(sv[2 * e] - m_ref), expf(sv[2 * e + 1] - m_ref));
                ls += __uint_as_float(pb[e] << 16) + __uint_as_float(pb[e] & 0xffff0000u);
            }
            ls += xor_lanes_f32<16>(ls);
            ls += xor_lanes_f32<32>(ls);
            l_run += ls;
            // O^T += V^T P^T, one MFMA per 32 rows: k-slots 0..3 <-> rows
            // 32*ks + 4*lg + e, 4..7 <-> rows 32*ks + 16 + 4*lg + e - 4 (the
            // lane's own S^T values of tiles 2*ks and 2*ks + 1)
#pragma unroll
            for (int ks = 0; ks < R / 32; ++ks) {
                bf16x8 pv;
                __builtin_memcpy(&pv, pb + 4 * ks, sizeof(pv));
#pragma unroll
                for (int md = 0; md < C::kMd; ++md) {
                    // column d = 16*md + li; row groups 8*ks + lg and 8*ks + 4 + lg
                    const int sw = pa_swz<R / 4>(2 * md);
                    const uint16_t* vr = vt + (16 * md + li) * C::kVtPitch;
                    const uint2 lo = *reinterpret_cast<const uint2*>(vr + 4 * ((8 * ks + lg) ^ sw));
                    const uint2 hi = *reinterpret_cast<const uint2*>(vr + 4 * ((8 * ks + 4 + lg) ^ sw));
                    const uint32_t wv4[4] = {lo.x, lo.y, hi.x, hi.y};
                    bf16x8 va;
                    __builtin_memcpy(&va, wv4, sizeof(va));
                    o[md] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pv, o[md], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }
    if (!active) return;
    // the sink joins the denominator once, at the end
    const int hh = 16 * wv + li;
    const float sk = a.sink ? a.sink[hh] : -INFINITY;
    const float M = fmaxf(m_ref, sk);
    const float em = expf(m_ref - M);
    const float es = sk == -INFINITY ? 0.f : expf(sk - M);
    const float den = l_run * em + es;
    const float f = em / den;
    if constexpr (kMixed) {  // columns 16 md + 4 lg + (0, 1) and (2, 3) are RoPE pairs past the NoPE part
        const float* cs = a.inv_cos + p * (kMixRope / 2);
        const float* sn = a.inv_sin + p * (kMixRope / 2);
#pragma unroll
        for (int md = kMixNope / 16; md < C::kMd; ++md) {
            const int pr = (16 * md + 4 * lg - kMixNope) / 2;
            float e0 = o[md][0], o0 = o[md][1], e1 = o[md][2], o1 = o[md][3];
            rope_pair(e0, o0, cs[pr], sn[pr], true);
            rope_pair(e1, o1, cs[pr + 1], sn[pr + 1], true);
            o[md] = f32x4{e0, o0, e1, o1};
        }
    }
    const long long ob = (static_cast<long long>(tq) * a.h + hh) * D + 4 * lg;
    if (a.out_bf16) {
#pragma unroll
        for (int md = 0; md < C::kMd; ++md) {
            const uint32_t x0 = bf16x2_rne(o[md][0] * f, o[md][1] * f);
            const uint32_t x1 = bf16x2_rne(o[md][2] * f, o[md][3] * f);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + ob + 16 * md) = make_uint2(x0, x1);
        }
    } else {
#pragma unroll
        for (int md = 0; md < C::kMd; ++md)
            *reinterpret_cast<float4*>(static_cast<float*>(a.out) + ob + 16 * md) =
                make_float4(o[md][0] * f, o[md][1] * f, o[md][2] * f, o[md][3] * f);
    }
    if (a.lse && lg == 0) a.lse[static_cast<long long>(tq) * a.h + hh] = M + logf(den);
}

template <int D>
size_t prefill_attn_lds(int k) {
    return PaCfg<D>::kLdsRows + sizeof(int) * static_cast<size_t>(k);
}

template <int D, bool kMixed = false>
hipError_t launch_prefill_attn_d(const PrefillAttnArgs& a, hipStream_t s) {
    const size_t lds = prefill_attn_lds<D>(a.k);
    if (lds > 64 * 1024) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
        static size_t opted[64] = {};
        if (opted[dev] < lds) {
            const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_prefill_attn<D, kMixed>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     static_cast<int>(prefill_attn_lds<D>(kTopkMaxK)));
            if (e != hipSuccess) return e;
            opted[dev] = prefill_attn_lds<D>(kTopkMaxK);
        }
    }
    hipLaunchKernelGGL((k_prefill_attn<D, kMixed>), dim3(a.t), dim3(kPaThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_index_score_mq(const ScoreArgs& sa, long long pos0, hipStream_t s) {
    if (sa.t <= 0 || sa.n <= 0 || sa.batch <= 0) return hipSuccess;
    const int groups = (sa.t + kMqRowsPerWg - 1) / kMqRowsPerWg;
    // one workgroup per CU in all; each key range is a whole number of 16-key tiles
    const long long per_split = static_cast<long long>(groups) * sa.batch;
    int splits = static_cast<int>((device_cu_count() + per_split - 1) / per_split);
    if (splits < 1) splits = 1;
    int kpw = (sa.n + splits - 1) / splits;
    kpw = (kpw + 15) / 16 * 16;
    splits = (sa.n + kpw - 1) / kpw;
    MqArgs a{static_cast<const uint16_t*>(sa.q), sa.w, static_cast<const uint16_t*>(sa.k), sa.scores, sa.t, sa.n,
             sa.ld_s, sa.q_pos, pos0, sa.ratio, kpw, sa.q_stride_b, sa.w_stride_b, sa.k_stride_b, sa.s_stride_b};
    if (kMqLds > 64 * 1024) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
        static bool opted[64] = {};
        if (!opted[dev]) {
            const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_index_score_mq<CSA_MQ_SHAPE>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     static_cast<int>(kMqLds));
            if (e != hipSuccess) return e;
            opted[dev] = true;
        }
    }
    hipLaunchKernelGGL((k_index_score_mq<CSA_MQ_SHAPE>), dim3(splits, groups, sa.batch), dim3(Mq::kThreads), kMqLds,
                       s, a);
    return hipGetLastError();
}

size_t index_topk_workspace_bytes(int t, int n, int top_k) {
    const int rows = t < kPrefillChunkRows ? t : kPrefillChunkRows;
    return pf_align256(sizeof(float) * static_cast<size_t>(rows) * (n > 0 ? n : 0)) +
           pf_align256(topk_workspace_bytes(rows, n, top_k));  // used only by rows over 65536 scores
}

hipError_t launch_index_topk(const IndexTopkArgs& a, hipStream_t s) {
    if (a.t <= 0) return hipSuccess;
    const int rows_max = a.t < kPrefillChunkRows ? a.t : kPrefillChunkRows;
    float* sc = static_cast<float*>(a.ws);
    void* tws = static_cast<char*>(a.ws) + pf_align256(sizeof(float) * static_cast<size_t>(rows_max) * a.n);
    for (int r0 = 0; r0 < a.t; r0 += kPrefillChunkRows) {
        const int rows = a.t - r0 < kPrefillChunkRows ? a.t - r0 : kPrefillChunkRows;
        const long long p0 = a.pos0 < 0 ? -1 : a.pos0 + r0;
        hipError_t e;
        if (a.k_scale) {
            Fp8ScoreArgs fa{};
            fa.q = a.q8 + static_cast<long long>(r0) * kIdxHeads * kIdxDi;
            fa.w = a.w + static_cast<long long>(r0) * kIdxHeads;
            fa.k = a.k8;
            fa.k_scale = a.k_scale;
            fa.k_fp4 = a.k_fp4;
            fa.scores = sc;
            fa.batch = 1;
            fa.t = rows;
            fa.n = a.n;
            fa.ratio = a.ratio;
            fa.ld_s = a.n;
            e = launch_index_score_mq_fp8(fa, p0, s);
        } else {
            ScoreArgs sa{};
            sa.q = a.q + static_cast<long long>(r0) * kIdxHeads * kIdxDi;
            sa.w = a.w + static_cast<long long>(r0) * kIdxHeads;
            sa.k = a.k;
            sa.scores = sc;
            sa.batch = 1;
            sa.t = rows;
            sa.h_i = kIdxHeads;
            sa.d_i = kIdxDi;
            sa.n = a.n;
            sa.ratio = a.ratio;
            sa.ld_s = a.n;
            e = launch_index_score_mq(sa, p0, s);
        }
        if (e != hipSuccess) return e;
        TopkArgs ta{};
        ta.scores = sc;
        ta.batch = 1;
        ta.t = rows;
        ta.n = a.n;
        ta.ld_s = a.n;
        ta.s_stride_b = 0;
        ta.k = a.top_k;
        ta.idx = a.idx + static_cast<long long>(r0) * a.top_k;
        ta.count = a.count ? a.count + r0 : nullptr;
        ta.ws = tws;
        e = launch_topk_rows(ta, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

bool prefill_attn_supported(int h, int d) {
    return h > 0 && h % 16 == 0 && h <= 16 * kPaWaves && (d == 128 || d == 256 || d == 512);
}

hipError_t launch_prefill_attn(const PrefillAttnArgs& a, hipStream_t s) {
    if (a.t <= 0) return hipSuccess;
    if (a.kv_mixed) return a.d == kMixD ? launch_prefill_attn_d<kMixD, true>(a, s) : hipErrorInvalidValue;
    switch (a.d) {
        case 128: return launch_prefill_attn_d<128>(a, s);
        case 256: return launch_prefill_attn_d<256>(a, s);
        case 512: return launch_prefill_attn_d<512>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace csa

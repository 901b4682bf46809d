// One split of the partial sparse attention, shared by the attention
// kernels (attn.hip) and the fused top-k + attention kernel of the decode
// step (step_attn.hip).  See attn.hip for the method and its sources.
#pragma once

#include "common.h"
#include "kernels.h"
#include "mixed_kv.h"

namespace csa {

namespace {

constexpr int kAttnThreads = 256;
constexpr int kHeadGroup = 16;

constexpr int kR = 32;               // rows per split: every thread issues all its row loads at once,
                                     // and short splits give more workgroups to spread the loads over
inline int attn_rows_per_split(int) { return kR; }
inline int attn_splits(int n_max) {
    const int r = attn_rows_per_split(n_max);
    return n_max > 0 ? (n_max + r - 1) / r : 1;
}

constexpr int kNt = kR / 16;         // 16-row MFMA tiles per split: waves 0 .. kNt-1 compute S
constexpr int kPPitch = kR + 8;      // LDS pitch of the probabilities

// LDS of one split (dynamic part): row tile [kR][d + 8], query group
// [16][d + 8], probabilities [16][kR + 8], all bf16.
__host__ __device__ inline size_t attn_split_lds_bytes(int d) {
    return sizeof(uint16_t) * (static_cast<size_t>(kR + kHeadGroup) * (d + 8) + kHeadGroup * kPPitch);
}

template <int NT>
struct AttnSplit {
    static constexpr int kWaves = NT / kWave;
    static constexpr int kQBatch = (kHeadGroup * 64 + NT - 1) / NT;  // query pieces per thread at d = 512
    static constexpr int kChunks = (kR * 64 + NT - 1) / NT;          // row pieces per thread at d = 512
    static_assert(kWaves >= kNt, "one wave per 16-row tile");
};

// The query group's loads (independent of everything else: issued first).
template <int NT>
__device__ inline void attn_load_q(const AttnArgs& a, int hg, int b, uint4 (&qv)[AttnSplit<NT>::kQBatch]) {
    const int d = a.d;
    const int cpr = d / 8;
    const uint16_t* qg = a.q + b * a.q_stride_b + static_cast<long long>(hg * kHeadGroup) * d;
#pragma unroll
    for (int u = 0; u < AttnSplit<NT>::kQBatch; ++u) {
        const int c = threadIdx.x + u * NT;
        qv[u] = c < kHeadGroup * cpr ? *reinterpret_cast<const uint4*>(qg + (c / cpr) * d + (c % cpr) * 8)
                                     : make_uint4(0, 0, 0, 0);
    }
}

// One split of the partial attention: rows [kR * split, kR * split + kR) of
// the gathered set (gather mode: top-k rows of the compressed cache, then the
// SWA window; dense mode: every compressed row in order, then the window) or
// of kv (plain mode), for the 16 heads of group hg.  Partial
// (m, l, O) go to the workspace.  rows_idx: this sequence's top-k indices
// (global or LDS); cnt_in: their count if known, else < 0 (read from
// a.count).  smem: attn_split_lds_bytes(d) of LDS.  Every thread calls it.
template <int NT>
__device__ inline void attn_split(const AttnArgs& a, int n_splits, int split, int hg, int b, const int* rows_idx,
                                  int cnt_in, const uint4 (&qv)[AttnSplit<NT>::kQBatch], uint16_t* smem) {
    using G = AttnSplit<NT>;
    __shared__ float wmax[kNt][kHeadGroup];
    __shared__ float wsum[kNt][kHeadGroup];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int d = a.d;
    const int pitch = d + 8;
    uint16_t* tile = smem;                        // [kR][d + 8]
    uint16_t* qs = tile + kR * pitch;             // [16][d + 8]
    uint16_t* pl = qs + kHeadGroup * pitch;       // [16][kR + 8]
    const int r0 = split * kR;
    const int cpr = d / 8;  // 16-byte chunks per row

    // valid rows (gather mode: top-k count + window).  The top-k index of
    // every row a thread's chunks fall in is read alongside the count, so
    // the row loads wait for one round trip only.
    const int n_chunks = kR * cpr;
    int my_idx[G::kChunks];
#pragma unroll
    for (int u = 0; u < G::kChunks; ++u) {
        const int c = u * NT + threadIdx.x;
        const int j = r0 + c / cpr;
        my_idx[u] = a.dense ? j : ((a.idx && c < n_chunks && j < a.k) ? rows_idx[j] : 0);
    }
    int cnt = 0, nv;
    if (a.idx || a.dense) {
        if (a.dense) {
            cnt = a.n_comp > 0 ? a.n_comp : 0;
        } else {
            cnt = cnt_in >= 0 ? cnt_in : (a.count ? a.count[b] : a.k);
            cnt = cnt < 0 ? 0 : (cnt > a.k ? a.k : cnt);
            if (a.n_comp <= 0) cnt = 0;
        }
        nv = cnt + a.swa_len;
        if (split == 0 && hg == 0 && threadIdx.x == 0 && a.n_valid_out) a.n_valid_out[b] = nv;
    } else {
        nv = a.n_valid[b];
    }
    nv = nv < 0 ? 0 : (nv > a.n_max ? a.n_max : nv);
    const int rows = max(0, min(kR, nv - r0));
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
    uint4 v[G::kChunks];
    if (a.kv_mixed) {
        // mixed records (d = 512): one 16-byte read and the row scale per chunk, with no branch on the
        // chunk kind (a load chosen between branches makes the compiler wait for it at the join);
        // chunks past the split's rows read the ring's first record.  Chunk cc < 56 decodes 8 codes
        // to bfloat16, chunk cc >= 56 is 16 bytes of the RoPE part.
        constexpr int kNopeChunks = kMixNope / 8;
        const uint8_t* cbase = reinterpret_cast<const uint8_t*>(a.comp_kv) + b * a.comp_kv_stride_b;
        const uint8_t* sbase = reinterpret_cast<const uint8_t*>(a.swa) + b * a.swa_stride_b;
        float vsc[G::kChunks];
#pragma unroll
        for (int u = 0; u < G::kChunks; ++u) {
            const int c = u * NT + threadIdx.x;
            const int r = c / cpr;
            const int j = r0 + r;
            const bool live = c < n_chunks && r < rows;
            int slot = (a.swa_head - a.swa_len + (j - cnt)) % a.w;
            if (slot < 0) slot += a.w;
            const int ri = my_idx[u] < 0 ? 0 : (my_idx[u] >= a.n_comp ? a.n_comp - 1 : my_idx[u]);
            const uint8_t* rec = !live ? sbase
                                       : (j < cnt ? cbase + static_cast<long long>(ri) * kMixRec
                                                  : sbase + static_cast<long long>(slot) * kMixRec);
            v[u] = mixed_piece_load(mixed_piece_ptr(rec, c % cpr));
            vsc[u] = *reinterpret_cast<const float*>(rec + kMixScaleOff);
        }
        const bool write_rec = a.idx && a.gather_buf && hg == 0;
        uint8_t* gbase = reinterpret_cast<uint8_t*>(a.gather_buf) + b * a.buf_stride_b;
#pragma unroll
        for (int u = 0; u < G::kChunks; ++u) {
            const int c = u * NT + threadIdx.x;
            const int r = c / cpr;
            const int cc = c % cpr;
            const bool live = c < n_chunks && r < rows;
            if (live && write_rec) {  // the record's own bytes to gather_buf
                uint8_t* out = gbase + static_cast<long long>(r0 + r) * kMixRec;
                if (cc < kNopeChunks) {
                    *reinterpret_cast<uint2*>(out + 8 * cc) = make_uint2(v[u].x, v[u].y);
                    if (cc == 0) *reinterpret_cast<uint4*>(out + kMixScaleOff) = make_uint4(__float_as_uint(vsc[u]), 0u, 0u, 0u);
                } else {
                    *reinterpret_cast<uint4*>(out + kMixNope + 16 * (cc - kNopeChunks)) = v[u];
                }
            }
            v[u] = live ? mixed_piece_value(v[u], vsc[u], cc) : make_uint4(0, 0, 0, 0);
        }
    } else {
#pragma unroll
    for (int u = 0; u < G::kChunks; ++u) {
        const int c = u * NT + threadIdx.x;
        const int r = c / cpr;
        const int j = r0 + r;
        const uint16_t* src = nullptr;
        if (c < n_chunks && r < rows) {
            if (!a.idx && !a.dense) {
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
    }
#pragma unroll
    for (int u = 0; u < G::kQBatch; ++u) {
        const int c = threadIdx.x + u * NT;
        if (c < kHeadGroup * cpr) *reinterpret_cast<uint4*>(qs + (c / cpr) * pitch + (c % cpr) * 8) = qv[u];
    }
    const bool write_buf = (a.idx || a.dense) && a.gather_buf && hg == 0 && !a.kv_mixed;
#pragma unroll
    for (int u = 0; u < G::kChunks; ++u) {
        const int c = u * NT + threadIdx.x;
        if (c < n_chunks) {
            const int r = c / cpr;
            const int cc = c % cpr;
            *reinterpret_cast<uint4*>(tile + r * pitch + cc * 8) = v[u];
            if (write_buf && r < rows)
                *reinterpret_cast<uint4*>(a.gather_buf + b * a.buf_stride_b + static_cast<long long>(r0 + r) * d + cc * 8) = v[u];
        }
    }
    __syncthreads();

    // 2. S = q K^T: wave wv < kNt owns rows 16*wv .. 16*wv+15
    const int li = lane & 15;
    const int lg = lane >> 4;
    const bool has_tile = wv < kNt;
    const int my_row = 16 * wv + li;
    float x[4];
    if (has_tile) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
        const uint16_t* qrow = qs + li * pitch + 8 * lg;
        const uint16_t* krow = tile + my_row * pitch + 8 * lg;
        const int nks = d / 32;
        int ks = 0;
        for (; ks + 4 <= nks; ks += 4) {  // four k-steps' operands in flight at once
            bf16x8 qa[4], kb[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                qa[u] = *reinterpret_cast<const bf16x8*>(qrow + 32 * (ks + u));
                kb[u] = *reinterpret_cast<const bf16x8*>(krow + 32 * (ks + u));
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[u], kb[u], s, 0, 0, 0);
        }
        for (; ks < nks; ++ks)
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(qrow + 32 * ks),
                                                        *reinterpret_cast<const bf16x8*>(krow + 32 * ks), s, 0,
                                                        0, 0);
        // accumulator register r <-> head 4*lg + r, row my_row
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = my_row < rows ? s[r] * a.scale : -INFINITY;
        // 3. split softmax: per-head max and sum over the rows (lanes, then the tile waves)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float m = x[r];
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, row16_xor(m, o));
            if (li == 0) wmax[wv][4 * lg + r] = m;
        }
    }
    __syncthreads();
    if (has_tile) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int hh = 4 * lg + r;
            float M = wmax[0][hh];
#pragma unroll
            for (int w = 1; w < kNt; ++w) M = fmaxf(M, wmax[w][hh]);
            // rows >= 1, so M is finite; masked rows give exp(-inf) = 0
            const uint16_t pb = f32_to_bf16(expf(x[r] - M));
            pl[hh * kPPitch + my_row] = pb;
            float e = bf16_to_f32(pb);
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) e += row16_xor(e, o);
            if (li == 0) wsum[wv][hh] = e;
        }
    }
    __syncthreads();
    if (threadIdx.x < kHeadGroup) {
        const int hh = threadIdx.x;
        float M = wmax[0][hh], l = wsum[0][hh];
#pragma unroll
        for (int w = 1; w < kNt; ++w) {
            M = fmaxf(M, wmax[w][hh]);
            l += wsum[w][hh];
        }
        a.ws_ml[2 * (ml_base + static_cast<long long>(hh) * n_splits) + 0] = M;
        a.ws_ml[2 * (ml_base + static_cast<long long>(hh) * n_splits) + 1] = l;
    }

    // 4. O = P V: M = 16 heads, K = kR rows (one MFMA step), N = d in 16-wide tiles
    float* ob = a.ws_o + (static_cast<long long>(b) * a.h + hg * kHeadGroup) * n_splits * d +
                static_cast<long long>(split) * d;
    for (int nt = wv; nt < d / 16; nt += G::kWaves) {
        const int col = 16 * nt + li;
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kR / 32; ++ks) {
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

}  // namespace

}  // namespace csa

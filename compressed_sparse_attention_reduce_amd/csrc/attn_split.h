// One split of the partial sparse attention, shared by the attention
// kernels (attn.hip) and the fused top-k + attention kernel of the decode
// step (step_attn.hip).  See attn.hip for the method and its sources.
#pragma once

#include <type_traits>

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

// Row and 16-byte chunk of the pieces c = threadIdx.x + u * NT (u < N) of a
// tile with cpr chunks per row: shifts and adds when NT is a multiple of cpr
// (power-of-two head dims), one division per piece otherwise.  (A division
// per piece is tens of instructions on every lane; across a tile's pieces it
// delays the issue of the row loads by microseconds.)
template <int NT, int N>
__device__ inline void piece_rows(int cpr, int (&r)[N], int (&p)[N]) {
    if (NT % cpr == 0) {
        const int rt = threadIdx.x / cpr;
        const int pt = threadIdx.x - rt * cpr;
        const int dr = NT / cpr;
#pragma unroll
        for (int u = 0; u < N; ++u) {
            r[u] = rt + u * dr;
            p[u] = pt;
        }
    } else {
#pragma unroll
        for (int u = 0; u < N; ++u) {
            const int c = threadIdx.x + u * NT;
            r[u] = c / cpr;
            p[u] = c - r[u] * cpr;
        }
    }
}

// Ring slot of window row i (0 = the oldest of the len live rows; 0 <= i <
// len <= w, head < w): head - len + i lies in (-w, w).
__device__ inline int swa_slot(int head, int len, int i, int w) {
    const int s = head - len + i;
    return s < 0 ? s + w : s;
}

// O = P V for a group of 16 * P columns of d starting at c_base (P = 2 or 4):
// M = 16 heads, K = rows in 32-row steps, N = columns.  Lane (li, lg) reads
// P adjacent columns (c_base + P li ..) of each of its 8 rows per step with
// one LDS read per row (4 or 8 bytes); byte permutes (v_perm_b32) regroup
// them into the B operands of P MFMAs (dword j: rows 2j and 2j + 1 of one
// column), so P MFMAs share 8 reads instead of taking 8 two-byte reads each.
// Accumulator t holds column c_base + P li + t; each head's P values leave as
// one store of P values of type Out to ob[head * ob_head_stride + column]:
// float32, or bfloat16 rounded to nearest even (Out = uint16_t, the HCA
// step's partials: half the bytes written here and read by its merge, a
// relative rounding of 2^-9 per partial on an output that is itself
// bfloat16).  Columns at or past d (a last, partial group) read column 0 and
// store nothing.
template <int P, typename Out = float>
__device__ inline void pv_group(const uint16_t* tile, int pitch, const uint16_t* pl, int ppitch, int ksteps,
                                int c_base, int d, Out* ob, long long ob_head_stride) {
    static_assert(P == 2 || P == 4, "two or four columns per lane");
    using Piece = typename std::conditional<P == 2, uint32_t, uint2>::type;
    const int lane = threadIdx.x & (kWave - 1);
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int cp = c_base + P * li;
    const bool cv = cp < d;
    const int cr = cv ? cp : 0;
    f32x4 o[P];
#pragma unroll
    for (int t = 0; t < P; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < ksteps; ++ks) {
        const bf16x8 pa = *reinterpret_cast<const bf16x8*>(pl + li * ppitch + 32 * ks + 8 * lg);
        Piece rv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) rv[e] = *reinterpret_cast<const Piece*>(tile + (32 * ks + 8 * lg + e) * pitch + cr);
#pragma unroll
        for (int t = 0; t < P; ++t) {
            const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;  // high or low halves
            uint32_t wd[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t lo, hi;
                if constexpr (P == 2) {
                    lo = rv[2 * j];
                    hi = rv[2 * j + 1];
                } else {
                    lo = t < 2 ? rv[2 * j].x : rv[2 * j].y;
                    hi = t < 2 ? rv[2 * j + 1].x : rv[2 * j + 1].y;
                }
                wd[j] = __builtin_amdgcn_perm(hi, lo, sel);
            }
            bf16x8 vb;
            __builtin_memcpy(&vb, wd, sizeof(vb));
            o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, o[t], 0, 0, 0);
        }
    }
    if (!cv) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        Out* dst = ob + static_cast<long long>(4 * lg + r) * ob_head_stride + cp;
        if constexpr (std::is_same<Out, float>::value) {
            if constexpr (P == 2)
                *reinterpret_cast<float2*>(dst) = make_float2(o[0][r], o[1][r]);
            else
                *reinterpret_cast<float4*>(dst) = make_float4(o[0][r], o[1][r], o[2][r], o[3][r]);
        } else {
            static_assert(std::is_same<Out, uint16_t>::value, "float32 or bfloat16 partials");
            const uint32_t w0 =
                static_cast<uint32_t>(f32_to_bf16(o[0][r])) | (static_cast<uint32_t>(f32_to_bf16(o[1][r])) << 16);
            if constexpr (P == 2) {
                *reinterpret_cast<uint32_t*>(dst) = w0;
            } else {
                const uint32_t w1 =
                    static_cast<uint32_t>(f32_to_bf16(o[2][r])) | (static_cast<uint32_t>(f32_to_bf16(o[3][r])) << 16);
                *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
            }
        }
    }
}

// Decode step with device counters: the step's view of them after its own
// jobs (the block it completes and the token's window row are in place);
// one workgroup records the position for the merge.  Returns the entry count.
__device__ inline int attn_dev_view(AttnArgs& a, bool record) {
    const DevState st = dev_load(a.dev, a.w, a.max_comp);
    if (record && a.dev_pos) *a.dev_pos = st.pos;
    const int n = dev_step_entries(st, a.m, a.max_comp);
    a.n_comp = n;
    a.swa_head = (st.swa_head + 1) % a.w;
    a.swa_len = st.swa_len + 1 < a.w ? st.swa_len + 1 : a.w;
    return n;
}

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
    int pr[G::kChunks], pc[G::kChunks];  // each piece's row of the split (kR and up: none) and chunk
    piece_rows<NT>(cpr, pr, pc);
    int my_idx[G::kChunks];
#pragma unroll
    for (int u = 0; u < G::kChunks; ++u) {
        const int j = r0 + pr[u];
        my_idx[u] = a.dense ? j : ((a.idx && pr[u] < kR && j < a.k) ? rows_idx[j] : 0);
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
    const bool direct = !a.kv_mixed && cpr == kWave && G::kChunks * (NT / kWave) == kR;
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
            const int j = r0 + pr[u];
            const bool live = pr[u] < rows;
            const int ri = my_idx[u] < 0 ? 0 : (my_idx[u] >= a.n_comp ? a.n_comp - 1 : my_idx[u]);
            const uint8_t* rec =
                !live ? sbase
                      : (j < cnt ? cbase + static_cast<long long>(ri) * kMixRec
                                 : sbase + static_cast<long long>(swa_slot(a.swa_head, a.swa_len, j - cnt, a.w)) *
                                               kMixRec);
            v[u] = mixed_piece_load(mixed_piece_ptr(rec, pc[u]));
            vsc[u] = *reinterpret_cast<const float*>(rec + kMixScaleOff);
        }
        const bool write_rec = a.idx && a.gather_buf && hg == 0;
        uint8_t* gbase = reinterpret_cast<uint8_t*>(a.gather_buf) + b * a.buf_stride_b;
#pragma unroll
        for (int u = 0; u < G::kChunks; ++u) {
            const int r = pr[u];
            const int cc = pc[u];
            const bool live = r < rows;
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
    } else if (direct) {
        // d = 512: piece u of wave wv is the whole row wv + u NT / 64 (lane =
        // chunk), so one wave instruction moves a row straight into its LDS
        // row (no registers, no LDS stores); rows past the split's are zeroed
        const int wvu = __builtin_amdgcn_readfirstlane(wv);
#pragma unroll
        for (int u = 0; u < G::kChunks; ++u) {
            const int r = wvu + u * (NT / kWave);
            const int j = r0 + r;
            if (r < rows) {
                const uint16_t* src;
                if (!a.idx && !a.dense) {
                    src = a.kv + b * a.kv_stride_b + static_cast<long long>(j) * d;
                } else if (j < cnt) {
                    const int ix = __builtin_amdgcn_readfirstlane(my_idx[u]);
                    const int ri = ix < 0 ? 0 : (ix >= a.n_comp ? a.n_comp - 1 : ix);
                    src = a.comp_kv + b * a.comp_kv_stride_b + static_cast<long long>(ri) * d;
                } else {
                    src = a.swa + b * a.swa_stride_b +
                          static_cast<long long>(swa_slot(a.swa_head, a.swa_len, j - cnt, a.w)) * d;
                }
                __builtin_amdgcn_global_load_lds(src + lane * 8,
                                                 (__attribute__((address_space(3))) void*)(tile + r * pitch), 16, 0,
                                                 0);
            } else {
                *reinterpret_cast<uint4*>(tile + r * pitch + lane * 8) = make_uint4(0, 0, 0, 0);
            }
        }
    } else {
#pragma unroll
    for (int u = 0; u < G::kChunks; ++u) {
        const int j = r0 + pr[u];
        const uint16_t* src = nullptr;
        if (pr[u] < rows) {
            if (!a.idx && !a.dense) {
                src = a.kv + b * a.kv_stride_b + static_cast<long long>(j) * d;
            } else if (j < cnt) {
                const int ri = my_idx[u] < 0 ? 0 : (my_idx[u] >= a.n_comp ? a.n_comp - 1 : my_idx[u]);
                src = a.comp_kv + b * a.comp_kv_stride_b + static_cast<long long>(ri) * d;
            } else {
                src = a.swa + b * a.swa_stride_b +
                      static_cast<long long>(swa_slot(a.swa_head, a.swa_len, j - cnt, a.w)) * d;
            }
        }
        v[u] = src ? *reinterpret_cast<const uint4*>(src + pc[u] * 8) : make_uint4(0, 0, 0, 0);
    }
    }
#pragma unroll
    for (int u = 0; u < G::kQBatch; ++u) {
        const int c = threadIdx.x + u * NT;
        if (c < kHeadGroup * cpr) *reinterpret_cast<uint4*>(qs + (c / cpr) * pitch + (c % cpr) * 8) = qv[u];
    }
    const bool write_buf = (a.idx || a.dense) && a.gather_buf && hg == 0 && !a.kv_mixed;
    if (direct) {
        __builtin_amdgcn_s_waitcnt(kVmcntZero);  // this wave's rows have landed in LDS
    } else {
#pragma unroll
        for (int u = 0; u < G::kChunks; ++u) {
            if (pr[u] < kR) {
                const int r = pr[u];
                const int cc = pc[u];
                *reinterpret_cast<uint4*>(tile + r * pitch + cc * 8) = v[u];
                if (write_buf && r < rows)
                    *reinterpret_cast<uint4*>(a.gather_buf + b * a.buf_stride_b + static_cast<long long>(r0 + r) * d +
                                              cc * 8) = v[u];
            }
        }
    }
    __syncthreads();
    if (direct && write_buf) {  // the wave's own rows, from LDS to gather_buf
#pragma unroll
        for (int u = 0; u < G::kChunks; ++u) {
            const int r = pr[u];
            if (r < rows)
                *reinterpret_cast<uint4*>(a.gather_buf + b * a.buf_stride_b + static_cast<long long>(r0 + r) * d +
                                          pc[u] * 8) = *reinterpret_cast<const uint4*>(tile + r * pitch + pc[u] * 8);
        }
    }

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
        if (d == 512) {  // all k-steps unrolled, two accumulators: half the dependent chain
            f32x4 s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k2 = 0; k2 < 16; k2 += 2) {
                s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(qrow + 32 * k2),
                                                            *reinterpret_cast<const bf16x8*>(krow + 32 * k2), s, 0, 0,
                                                            0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(qrow + 32 * k2 + 32),
                                                             *reinterpret_cast<const bf16x8*>(krow + 32 * k2 + 32), s1,
                                                             0, 0, 0);
            }
            s += s1;
            ks = nks;
        }
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

    // 4. O = P V: M = 16 heads, K = kR rows, N = d in groups of 16 P columns
    //    (P = 2 when the waves are many, so every wave gets a group at d = 512)
    float* ob = a.ws_o + (static_cast<long long>(b) * a.h + hg * kHeadGroup) * n_splits * d +
                static_cast<long long>(split) * d;
    constexpr int kP = G::kWaves >= 16 ? 2 : 4;
    for (int g = wv; 16 * kP * g < d; g += G::kWaves)
        pv_group<kP>(tile, pitch, pl, kPPitch, kR / 32, 16 * kP * g, d, ob, static_cast<long long>(n_splits) * d);
}

}  // namespace

}  // namespace csa

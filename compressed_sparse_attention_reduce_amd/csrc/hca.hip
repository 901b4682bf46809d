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
// of 32-row splits, and k_attn_merge_rows merges them.  The partial outputs
// are stored in bfloat16 (the (max, sum) pairs in float32), halving what the
// attention writes and the merge reads again.  The four head groups
// of a split run on one XCD (consecutive workgroup ids go to consecutive
// XCDs), so the rows come from HBM once and from that XCD's L2 for the other
// three groups.  One workgroup per split and head group and nothing else
// (the step's SWA append aside), so that every workgroup is resident at
// once: a ratio-m block the step completes is compressed by the attention
// workgroups themselves, a slice of channels each.
#include "attn_split.h"
#include "common.h"
#include "kernels.h"
#include "mixed_kv.h"
#include "step_prep.h"

namespace csa {

namespace {

constexpr int kDenseThreads = 512;
constexpr int kDenseWaves = kDenseThreads / kWave;
constexpr int kDenseRows = 16 * kDenseWaves;          // rows per split: one 16-row S tile per wave
constexpr int kDensePPitch = kDenseRows + 8;          // LDS pitch of the probabilities
constexpr int kDenseMaxD = 512;
constexpr int kDenseQPer = kHeadGroup * kDenseMaxD / 8 / kDenseThreads;  // query pieces per thread
constexpr int kDenseRowPer = kDenseRows * kDenseMaxD / 8 / kDenseThreads; // row pieces per thread
// channels of a folded block compression per workgroup, at least: 32 row
// slices of 4 rows each for a 128-row block, merged by 16 threads
constexpr int kFoldMinCh = 16;
constexpr int kFoldPre = 4;  // rows of its slice a thread loads with the attention's rows (a 128-row block)

// The slices' (max, denominator, weighted sum) of the folded compression
// combined: transposed through LDS so that a channel's slices sit in
// consecutive lanes, the channel's maximum by lane swaps, each slice rescaled
// to it once, then the sums by lane swaps; y = sum / denominator.  Other
// slice counts take slice_merge.  part: 3 * blockDim.x floats of LDS.
__device__ inline void fold_merge(float mx, float den, float acc, void* __restrict__ out_row, bool out_bf16, int d,
                                  int ch0, int nch, float* part) {
    const int slices = blockDim.x / nch;
    if ((slices & (slices - 1)) != 0 || slices > kWave || slices * nch != static_cast<int>(blockDim.x)) {
        slice_merge(mx, den, acc, out_row, out_bf16, d, ch0, nch, part);
        return;
    }
    part[threadIdx.x] = mx;
    part[blockDim.x + threadIdx.x] = den;
    part[2 * blockDim.x + threadIdx.x] = acc;
    __syncthreads();
    const int tc = threadIdx.x / slices;
    const int s2 = threadIdx.x % slices;
    const float m2 = part[s2 * nch + tc];
    float d2 = part[blockDim.x + s2 * nch + tc];
    float a2 = part[2 * blockDim.x + s2 * nch + tc];
    float M = m2;
    if (slices > 1) M = fmaxf(M, xor_lanes_f32<1>(M));
    if (slices > 2) M = fmaxf(M, xor_lanes_f32<2>(M));
    if (slices > 4) M = fmaxf(M, xor_lanes_f32<4>(M));
    if (slices > 8) M = fmaxf(M, xor_lanes_f32<8>(M));
    if (slices > 16) M = fmaxf(M, xor_lanes_f32<16>(M));
    if (slices > 32) M = fmaxf(M, xor_lanes_f32<32>(M));
    const float f = m2 == -INFINITY ? 0.f : expf(m2 - M);  // an empty slice adds nothing
    d2 *= f;
    a2 *= f;
    if (slices > 1) { d2 += xor_lanes_f32<1>(d2); a2 += xor_lanes_f32<1>(a2); }
    if (slices > 2) { d2 += xor_lanes_f32<2>(d2); a2 += xor_lanes_f32<2>(a2); }
    if (slices > 4) { d2 += xor_lanes_f32<4>(d2); a2 += xor_lanes_f32<4>(a2); }
    if (slices > 8) { d2 += xor_lanes_f32<8>(d2); a2 += xor_lanes_f32<8>(a2); }
    if (slices > 16) { d2 += xor_lanes_f32<16>(d2); a2 += xor_lanes_f32<16>(a2); }
    if (slices > 32) { d2 += xor_lanes_f32<32>(d2); a2 += xor_lanes_f32<32>(a2); }
    if (s2 == 0 && ch0 + tc < d) {
        const float y = a2 / d2;
        if (out_bf16)
            static_cast<uint16_t*>(out_row)[ch0 + tc] = f32_to_bf16(y);
        else
            static_cast<float*>(out_row)[ch0 + tc] = y;
    }
}

__host__ __device__ inline size_t dense_lds_bytes(int d) {
    return sizeof(uint16_t) * (static_cast<size_t>(kDenseRows + kHeadGroup) * (d + 8) +
                               static_cast<size_t>(kHeadGroup) * kDensePPitch);
}

// mixed: the rows are mixed records (mixed_kv.h), decoded to bfloat16 on
// load, and the folded compression writes the block's entry in float32 to
// entry_f32 ([B][512]) for the merge to pack.
__global__ __launch_bounds__(kDenseThreads) void k_attn_dense_bf16(AttnArgs a, int n_splits, int prep_wgs, PrepArgs p,
                                                                    int extra_rows, int fold_ch, float* entry_f32) {
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    __shared__ __attribute__((aligned(16))) float wmax[kDenseWaves][kHeadGroup];
    __shared__ float wsum[kDenseWaves][kHeadGroup];
    // the step's small jobs (SWA append, compression of a completed block) in
    // their own workgroups; the rows they write are not
    // read here (the attention covers the rows before the step, the merge
    // adds the two new ones)
    // (first in the grid, so they start before the attention fills the CUs)
    if (static_cast<int>(blockIdx.x) < prep_wgs) {
        step_prep_role(p, blockIdx.x, blockIdx.y, reinterpret_cast<float*>(smem), &wmax[0][0]);
        return;
    }
    const int groups = a.h / kHeadGroup;
    // workgroup id -> (split, head group): over the first 8 * (n_splits / 8)
    // splits id % 8 = split % 8, so a split's head groups share an XCD; the
    // remaining splits follow one after another
    const int id = blockIdx.x - prep_wgs;
    const int n_full = n_splits / 8 * 8;
    int split, hg;
    if (id < n_full * groups) {
        const int rest = id / 8;
        hg = rest % groups;
        split = id % 8 + 8 * (rest / groups);
    } else {
        split = n_full + (id - n_full * groups) / groups;
        hg = (id - n_full * groups) % groups;
    }
    const int b = blockIdx.y;
    // device counters: the step's view of them (before its own append), and
    // the record the merge reads instead of the state
    bool dev_done = true;  // (host counters: whether a block completes is known on the host)
    if (a.dev) {
        const DevState st = dev_load(a.dev, a.w, a.max_comp);
        dev_done = dev_completes(st, a.m, a.max_comp);
        p.completes = dev_done ? 1 : 0;
        p.n_comp = st.n_comp;
        p.block = st.pos / a.m;
        a.n_comp = st.n_comp;
        a.swa_head = st.swa_head;
        a.swa_len = (st.swa_len + 1 < a.w ? st.swa_len + 1 : a.w) - 1;
        extra_rows = 1 + (dev_done ? 1 : 0);
        if (a.dev_pos && id == 0 && b == 0 && threadIdx.x == 0) {
            a.dev_pos[0] = st.pos;
            a.dev_pos[1] = st.n_comp;
            a.dev_pos[2] = dev_done ? 1 : 0;
        }
    }
    // A block this step completes is compressed here, fold_ch channels per
    // workgroup by the first ones (ratio-m blocks are long: one workgroup
    // alone would take longer than the attention).  Its rows are independent
    // of the attention's, which covers the entries before the step only, so
    // the channels' inputs are loaded with the attention's rows and reduced
    // after the partials are written.  With device counters the block's last
    // row is the token's own; the others come from the ring, to which each
    // folding workgroup adds its channels of the token's row.
    const bool fold = fold_ch > 0 && id * fold_ch < p.d && dev_done;  // uniform
    const int f_ch0 = id * fold_ch;
    const int f_nch = fold ? min(fold_ch, p.d - f_ch0) : 0;
    int f_ch = 0, f_lo = 0, f_hi = 0;
    float fz[kFoldPre], fb[kFoldPre], fc[kFoldPre];
    const float* f_z = p.z_main + b * p.zc_main_stride_b;
    const float* f_c = p.c_main + b * p.zc_main_stride_b;
    auto fold_src = [&](int r, const float*& zr, const float*& cr) {
        if (p.dev && r < p.m - 1) {
            const float* rz = p.dev_ring + b * p.ring_stride_b;
            const long long o = (p.block & 1) * static_cast<long long>(p.m) * p.d + static_cast<long long>(r) * p.d;
            zr = rz + o;
            cr = rz + 2LL * p.m * p.d + o;
        } else if (p.dev) {
            zr = f_z;
            cr = f_c;
        } else {
            zr = f_z + static_cast<long long>(r) * p.d;
            cr = f_c + static_cast<long long>(r) * p.d;
        }
    };
    auto fold_load = [&]() {
        slice_rows(p.m, p.d, f_ch0, f_nch, f_ch, f_lo, f_hi);
#pragma unroll
        for (int u = 0; u < kFoldPre; ++u) {
            const int r = f_lo + u;
            fz[u] = fb[u] = fc[u] = 0.f;
            if (r < f_hi) {
                const float* zr;
                const float* cr;
                fold_src(r, zr, cr);
                fz[u] = zr[f_ch];
                fb[u] = p.main_bias[static_cast<long long>(r) * p.d + f_ch];
                fc[u] = cr[f_ch];
            }
        }
    };
    // every thread calls it (scratch: 3 * blockDim.x floats of LDS, free)
    auto fold_finish = [&](float* scratch) {
        // the loaded rows against their own maximum (one exponential per row),
        // any further rows of a longer slice by the running form
        float lz[kFoldPre];
        float mx = -INFINITY, den = 0.f, acc = 0.f;
#pragma unroll
        for (int u = 0; u < kFoldPre; ++u) {
            lz[u] = fz[u] + fb[u];
            if (f_lo + u < f_hi) mx = fmaxf(mx, lz[u]);
        }
#pragma unroll
        for (int u = 0; u < kFoldPre; ++u) {
            if (f_lo + u < f_hi) {
                const float e = expf(lz[u] - mx);
                den += e;
                acc += e * fc[u];
            }
        }
        for (int r = f_lo + kFoldPre; r < f_hi; ++r) {
            const float* zr;
            const float* cr;
            fold_src(r, zr, cr);
            slice_row_update(zr[f_ch] + p.main_bias[static_cast<long long>(r) * p.d + f_ch], cr[f_ch], mx, den, acc);
        }
        if (p.dev) {  // the token's channels into the ring (its slot in the block's half)
            float* rz = p.dev_ring + b * p.ring_stride_b;
            const long long o = ((p.block & 1) * static_cast<long long>(p.m) + p.m - 1) * p.d + f_ch0;
            for (int j = threadIdx.x; j < f_nch; j += blockDim.x) {
                rz[o + j] = f_z[f_ch0 + j];
                rz[2LL * p.m * p.d + o + j] = f_c[f_ch0 + j];
            }
        }
        void* out = entry_f32 ? static_cast<void*>(entry_f32 + static_cast<long long>(b) * p.d)
                              : static_cast<void*>(static_cast<char*>(p.comp_kv) +
                                                   (b * p.comp_kv_stride_b + static_cast<long long>(p.n_comp) * p.d) *
                                                       p.es);
        fold_merge(mx, den, acc, out, !entry_f32 && p.es == 2, p.d, f_ch0, f_nch, scratch);
    };
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
    if (split == 0 && hg == 0 && threadIdx.x == 0 && a.n_valid_out) a.n_valid_out[b] = nv + extra_rows;
    if (rows == 0) {
        if (threadIdx.x < kHeadGroup) {
            a.ws_ml[2 * (ml_base + static_cast<long long>(threadIdx.x) * n_splits) + 0] = -INFINITY;
            a.ws_ml[2 * (ml_base + static_cast<long long>(threadIdx.x) * n_splits) + 1] = 0.f;
        }
        if (fold) {
            fold_load();
            fold_finish(reinterpret_cast<float*>(smem));
        }
        return;
    }
    // 1. the split's rows and the query group to LDS, all loads in one batch
    const uint16_t* qg = a.q + b * a.q_stride_b + static_cast<long long>(hg * kHeadGroup) * d;
    const uint16_t* comp = a.comp_kv + b * a.comp_kv_stride_b;
    const uint16_t* swa = a.swa + b * a.swa_stride_b;
    uint4 qv[kDenseQPer], v[kDenseRowPer];
    float vsc[kDenseRowPer];  // mixed: the row scale of each piece
    int pr[kDenseRowPer], pc[kDenseRowPer];  // each piece's row of the split (kDenseRows and up: none) and chunk
    piece_rows<kDenseThreads>(cpr, pr, pc);
    // d = 512: piece u of wave wv is the whole row wv + 8 u (lane = chunk), so
    // the row, its source and its bounds test are wave-uniform (scalar) and a
    // load costs one address add
    const bool wave_rows = cpr == kWave;
    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    constexpr int kRowStep = kDenseThreads / kWave;
    if (a.kv_mixed) {  // records (d = 512): one 16-byte read and the row scale per piece, no branch on the
                       // piece kind; pieces past the split's rows read its first row (rows >= 1)
        const uint8_t* cbase = reinterpret_cast<const uint8_t*>(a.comp_kv) + b * a.comp_kv_stride_b;
        const uint8_t* sbase = reinterpret_cast<const uint8_t*>(a.swa) + b * a.swa_stride_b;
        auto rec_of = [&](int jj) {
            return jj < cnt ? cbase + static_cast<long long>(jj) * kMixRec
                            : sbase + static_cast<long long>(swa_slot(a.swa_head, a.swa_len, jj - cnt, a.w)) * kMixRec;
        };
        if (wave_rows) {
#pragma unroll
            for (int u = 0; u < kDenseRowPer; ++u) {
                const int r = wvu + u * kRowStep;
                const uint8_t* rec = rec_of(r < rows ? r0 + r : r0);
                v[u] = mixed_piece_load(mixed_piece_ptr(rec, lane));
                vsc[u] = *reinterpret_cast<const float*>(rec + kMixScaleOff);
            }
        } else {
#pragma unroll
            for (int u = 0; u < kDenseRowPer; ++u) {
                const uint8_t* rec = rec_of(pr[u] < rows ? r0 + pr[u] : r0);
                v[u] = mixed_piece_load(mixed_piece_ptr(rec, pc[u]));
                vsc[u] = *reinterpret_cast<const float*>(rec + kMixScaleOff);
            }
        }
    } else {
        auto row_of = [&](int j) {
            return j < cnt ? comp + static_cast<long long>(j) * d
                           : swa + static_cast<long long>(swa_slot(a.swa_head, a.swa_len, j - cnt, a.w)) * d;
        };
        if (wave_rows) {
            // one whole row per wave instruction, straight into its LDS row
            // (no registers, no LDS stores); rows past the split's repeat its
            // first row, whose probabilities are zero
#pragma unroll
            for (int u = 0; u < kDenseRowPer; ++u) {
                const int r = wvu + u * kRowStep;
                __builtin_amdgcn_global_load_lds(row_of(r < rows ? r0 + r : r0) + lane * 8,
                                                 (__attribute__((address_space(3))) void*)(tile + r * pitch), 16, 0,
                                                 0);
            }
        } else {
#pragma unroll
            for (int u = 0; u < kDenseRowPer; ++u)
                v[u] = pr[u] < rows ? *reinterpret_cast<const uint4*>(row_of(r0 + pr[u]) + pc[u] * 8)
                                    : make_uint4(0, 0, 0, 0);
        }
    }
#pragma unroll
    for (int u = 0; u < kDenseQPer; ++u) {  // the query group after the rows (used only at the LDS staging)
        const int c = threadIdx.x + u * kDenseThreads;
        qv[u] = c < kHeadGroup * cpr ? *reinterpret_cast<const uint4*>(qg + (c / cpr) * d + (c % cpr) * 8)
                                     : make_uint4(0, 0, 0, 0);
    }
    // the block's channels: loads behind the rows', reduced at the end
    if (fold) fold_load();
    if (a.kv_mixed) {  // decode the pieces (the first use of the loaded bytes); rows past the split's are zero
#pragma unroll
        for (int u = 0; u < kDenseRowPer; ++u)
            v[u] = pr[u] < rows ? mixed_piece_value(v[u], vsc[u], pc[u]) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kDenseQPer; ++u) {
        const int c = threadIdx.x + u * kDenseThreads;
        if (c < kHeadGroup * cpr) *reinterpret_cast<uint4*>(qs + (c / cpr) * pitch + (c % cpr) * 8) = qv[u];
    }
    const bool direct = wave_rows && !a.kv_mixed;  // the rows went straight to LDS
    if (direct) {
        __builtin_amdgcn_s_waitcnt(kVmcntZero);  // this wave's row loads have landed
    } else {
#pragma unroll
        for (int u = 0; u < kDenseRowPer; ++u)
            if (pr[u] < kDenseRows) *reinterpret_cast<uint4*>(tile + pr[u] * pitch + pc[u] * 8) = v[u];
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
        if (d == kDenseMaxD) {  // all k-steps unrolled, two accumulators: half the dependent chain
            f32x4 s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k2 = 0; k2 < kDenseMaxD / 32; k2 += 2) {
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(qrow + 32 * k2),
                                                               *reinterpret_cast<const bf16x8*>(krow + 32 * k2), sacc,
                                                               0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(qrow + 32 * k2 + 32),
                                                             *reinterpret_cast<const bf16x8*>(krow + 32 * k2 + 32), s1,
                                                             0, 0, 0);
            }
            sacc += s1;
            ks = nks;
        }
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
    float Mr[4];  // the split's maximum of heads 4 lg .. 4 lg + 3: one 16-byte read per wave
    {
        float4 m4 = *reinterpret_cast<const float4*>(&wmax[0][4 * lg]);
#pragma unroll
        for (int w = 1; w < kDenseWaves; ++w) {
            const float4 o = *reinterpret_cast<const float4*>(&wmax[w][4 * lg]);
            m4.x = fmaxf(m4.x, o.x); m4.y = fmaxf(m4.y, o.y); m4.z = fmaxf(m4.z, o.z); m4.w = fmaxf(m4.w, o.w);
        }
        Mr[0] = m4.x; Mr[1] = m4.y; Mr[2] = m4.z; Mr[3] = m4.w;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int hh = 4 * lg + r;
        const float M = Mr[r];
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
    // 4. O = P V: M = 16 heads, K = the split's rows in 32-row steps, N = d in
    //    groups of 64 columns, one per wave
    uint16_t* ob = reinterpret_cast<uint16_t*>(a.ws_o) + (static_cast<long long>(b) * a.h + hg * kHeadGroup) * n_splits * d +
                   static_cast<long long>(split) * d;
    const int ksteps = (rows + 31) / 32;  // rows past the valid ones hold zeros and p = 0
    for (int g = wv; 64 * g < d; g += kDenseWaves)
        pv_group<4, uint16_t>(tile, pitch, pl, kDensePPitch, ksteps, 64 * g, d, ob, static_cast<long long>(n_splits) * d);
    if (fold) {
        __syncthreads();  // P V's reads of the tile are over: it becomes the merge's scratch
        fold_finish(reinterpret_cast<float*>(smem));
    }
}

// Merge of the splits plus the step's new rows (the compressed entry of a
// completed block, x0, if any; the new token's KV row, x1), one workgroup per
// (head, 128 columns, sequence): M = max of the splits' maxima, the new rows'
// logits and the sink; out = (sum_s e^(m_s - M) O_s + sum_i e^(s_i - M) x_i)
// / den with den = sum_s e^(m_s - M) l_s + sum_i e^(s_i - M) + e^(sink - M).
// At most 64 splits (lane s of every wave holds split s's (m, l)).  Wave w
// sums splits w, w + 4, ... for its 64 column pairs; the four partial sums
// meet in LDS.
constexpr int kMergeThreads = 256;
constexpr int kMergeWaves = kMergeThreads / kWave;
constexpr int kMergeCols = 2 * kWave;  // columns per workgroup: a column pair per lane
// Mixed main KV (a.kv_mixed, d = 512): x0f is the new entry in float32
// ([B][512], from the attention kernel, or nullptr) and x1 the new token's
// row; both take part as the caches now hold them (packed, then decoded as
// the attention's loader decodes), and workgroup 0 of each sequence writes
// the entry's record to rec0 (entry_cos / entry_sin: its RoPE row); the
// output's RoPE dims are rotated back with a.inv_cos / a.inv_sin.
__global__ __launch_bounds__(kMergeThreads) void k_attn_merge_rows(AttnArgs a, int n_splits, const uint16_t* x0,
                                                                   long long x0_stride_b, const uint16_t* x1,
                                                                   long long x1_stride_b, const float* x0f,
                                                                   uint8_t* rec0, long long rec0_stride_b,
                                                                   const float* entry_cos, const float* entry_sin) {
    __shared__ float red[2][kMergeWaves];
    __shared__ float2 part[kMergeWaves][kWave];
    __shared__ float xv[2][kMixD];  // mixed: the new rows' values as stored
    const int d = a.d;
    if (a.dev) {
        // device counters: the attention launch recorded (pos, n_comp,
        // completes) as the step saw them; the new entry (if any), its
        // record and the RoPE rows follow from it
        const int pos = a.dev_pos[0];
        const int n0 = a.dev_pos[1];
        const bool done = a.dev_pos[2] != 0;
        if (!done) {
            x0 = nullptr;
            x0f = nullptr;
            rec0 = nullptr;
        } else if (a.kv_mixed) {
            rec0 = const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(a.comp_kv)) + static_cast<long long>(n0) * kMixRec;
        } else {
            x0 = a.comp_kv + static_cast<long long>(n0) * d;
        }
        if (a.kv_mixed) {
            const int blk = pos / a.m < a.comp_rope_rows ? pos / a.m : a.comp_rope_rows - 1;
            entry_cos = a.comp_rope_cos + static_cast<long long>(blk) * (kMixRope / 2);
            entry_sin = a.comp_rope_sin + static_cast<long long>(blk) * (kMixRope / 2);
            const int pr = pos < a.rope_rows ? pos : a.rope_rows - 1;
            a.inv_cos = a.rope_cos + static_cast<long long>(pr) * (kMixRope / 2);
            a.inv_sin = a.rope_sin + static_cast<long long>(pr) * (kMixRope / 2);
        }
    }
    const int col_blocks = (d + kMergeCols - 1) / kMergeCols;
    const int hh = blockIdx.x / col_blocks;
    const int cb = blockIdx.x % col_blocks;
    const int b = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const long long base = (static_cast<long long>(b) * a.h + hh) * n_splits;
    const uint16_t* ob = reinterpret_cast<const uint16_t*>(a.ws_o) + base * d;
    // this wave's splits for the workgroup's columns and the splits' (m, l),
    // loaded first so that they are in flight with the new rows' loads; empty
    // splits' slots hold stale bytes, selected away (never multiplied)
    const int col2 = cb * kMergeCols + 2 * lane;
    const bool has_col = col2 < d;
    constexpr int kBatch = 16;
    float2 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
        const int sp = wv + kMergeWaves * u;
        const uint32_t w = (has_col && sp < n_splits) ? *reinterpret_cast<const uint32_t*>(ob + static_cast<long long>(sp) * d + col2)
                                                      : 0u;
        v[u] = make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
    }
    const float ms = lane < n_splits ? a.ws_ml[2 * (base + lane)] : -INFINITY;
    const float ls = lane < n_splits ? a.ws_ml[2 * (base + lane) + 1] : 0.f;
    // the new rows' logits: q . x_i over the whole head, two sums at once
    // (d <= 2 * kMergeThreads)
    const uint16_t* qh = a.q + b * a.q_stride_b + static_cast<long long>(hh) * d;
    const uint16_t* x0b = x0 ? x0 + b * x0_stride_b : nullptr;
    const uint16_t* x1b = x1 + b * x1_stride_b;
    auto pair = [](const uint16_t* p, int c, float& lo, float& hi) {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(p + c);
        lo = __uint_as_float(v << 16);
        hi = __uint_as_float(v & 0xffff0000u);
    };
    float d0 = 0.f, d1 = 0.f;
    if (a.kv_mixed) {
        // the new rows packed as the caches hold them: E4M3 NoPE with the
        // row's scale (block maxima first), bf16 RoPE (the entry rotated)
        const int col = 2 * threadIdx.x;  // d = 512: every column pair once
        float q0, q1, u0 = 0.f, u1 = 0.f, v0, v1;
        pair(qh, col, q0, q1);
        if (x0f) {
            u0 = x0f[static_cast<long long>(b) * kMixD + col];
            u1 = x0f[static_cast<long long>(b) * kMixD + col + 1];
        }
        pair(x1b, col, v0, v1);
        const bool nope = col < kMixNope;
        float m0 = nope ? fmaxf(fabsf(u0), fabsf(u1)) : 0.f;
        float m1 = nope ? fmaxf(fabsf(v0), fabsf(v1)) : 0.f;
        m0 = wave_max(m0);
        m1 = wave_max(m1);
        if (lane == 0) {
            red[0][wv] = m0;
            red[1][wv] = m1;
        }
        __syncthreads();
        m0 = red[0][0];
        m1 = red[1][0];
#pragma unroll
        for (int w = 1; w < kMergeWaves; ++w) {
            m0 = fmaxf(m0, red[0][w]);
            m1 = fmaxf(m1, red[1][w]);
        }
        __syncthreads();  // red is reused for the logits
        const float s0 = m0 > 0.f ? m0 / 448.0f : 1.0f;
        const float s1 = m1 > 0.f ? m1 / 448.0f : 1.0f;
        uint8_t* rec = (rec0 && blockIdx.x == 0) ? rec0 + b * rec0_stride_b : nullptr;
        if (nope) {
            const uint8_t c0 = e4m3_encode_rne(u0 / s0), c1 = e4m3_encode_rne(u1 / s0);
            u0 = bf16_round(e4m3_decode(c0) * s0);
            u1 = bf16_round(e4m3_decode(c1) * s0);
            v0 = bf16_round(e4m3_decode(e4m3_encode_rne(v0 / s1)) * s1);
            v1 = bf16_round(e4m3_decode(e4m3_encode_rne(v1 / s1)) * s1);
            if (rec && x0f) {
                rec[col] = c0;
                rec[col + 1] = c1;
            }
        } else {
            u0 = bf16_round(u0);
            u1 = bf16_round(u1);
            const int pr = (col - kMixNope) / 2;
            if (x0f) {
                rope_pair(u0, u1, entry_cos[pr], entry_sin[pr], false);
                u0 = bf16_round(u0);
                u1 = bf16_round(u1);
            }
            if (rec && x0f)
                *reinterpret_cast<uint32_t*>(rec + kMixNope + 4 * pr) =
                    static_cast<uint32_t>(f32_to_bf16(u0)) | (static_cast<uint32_t>(f32_to_bf16(u1)) << 16);
        }
        if (rec && x0f && threadIdx.x == 0)
            *reinterpret_cast<uint4*>(rec + kMixScaleOff) = make_uint4(__float_as_uint(s0), 0u, 0u, 0u);
        xv[0][col] = u0;
        xv[0][col + 1] = u1;
        xv[1][col] = v0;
        xv[1][col + 1] = v1;
        d0 = q0 * u0 + q1 * u1;
        d1 = q0 * v0 + q1 * v1;
    } else {
        const int col = 2 * threadIdx.x;
        if (col < d) {
            float q0, q1, u0 = 0.f, u1 = 0.f, v0, v1;
            pair(qh, col, q0, q1);
            if (x0b) pair(x0b, col, u0, u1);
            pair(x1b, col, v0, v1);
            d0 = q0 * u0 + q1 * u1;
            d1 = q0 * v0 + q1 * v1;
        }
    }
    d0 = wave_sum(d0);
    d1 = wave_sum(d1);
    if (lane == 0) {
        red[0][wv] = d0;
        red[1][wv] = d1;
    }
    float M = wave_max(ls > 0.f ? ms : -INFINITY);
    __syncthreads();
    d0 = 0.f;
    d1 = 0.f;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) {
        d0 += red[0][w];
        d1 += red[1][w];
    }
    const bool has_x0 = x0 != nullptr || x0f != nullptr;
    const float s0 = has_x0 ? d0 * a.scale : -INFINITY;
    const float s1 = d1 * a.scale;
    M = fmaxf(M, fmaxf(s0, s1));
    const float sk = a.sink ? a.sink[hh] : -INFINITY;
    M = fmaxf(M, sk);  // finite: s1 is
    const float wsp = ls > 0.f ? expf(ms - M) : 0.f;
    float acc0 = 0.f, acc1 = 0.f;
    static_assert(kMergeWaves * kBatch >= kWave, "one batch covers every split");
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
        const int sp = wv + kMergeWaves * u;
        const float c = sp < n_splits ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wsp), sp < kWave ? sp : 0))
                                      : 0.f;
        acc0 += c != 0.f ? c * v[u].x : 0.f;
        acc1 += c != 0.f ? c * v[u].y : 0.f;
    }
    part[wv][lane] = make_float2(acc0, acc1);
    __syncthreads();
    if (wv != 0) return;
    const float e0 = has_x0 ? expf(s0 - M) : 0.f;
    const float e1 = expf(s1 - M);
    const float es = a.sink ? expf(sk - M) : 0.f;
    const float den = wave_sum(wsp * ls) + e0 + e1 + es;
    const float inv = 1.0f / den;
    if (has_col) {
        float u0 = 0.f, u1 = 0.f, w0, w1;
        if (a.kv_mixed) {
            u0 = xv[0][col2];
            u1 = xv[0][col2 + 1];
            w0 = xv[1][col2];
            w1 = xv[1][col2 + 1];
        } else {
            if (x0b) pair(x0b, col2, u0, u1);
            pair(x1b, col2, w0, w1);
        }
        float o0 = e0 * u0 + e1 * w0, o1 = e0 * u1 + e1 * w1;
#pragma unroll
        for (int w = 0; w < kMergeWaves; ++w) {
            o0 += part[w][lane].x;
            o1 += part[w][lane].y;
        }
        o0 *= inv;
        o1 *= inv;
        // mixed KV: the RoPE dims rotated back at the token's position
        if (a.inv_cos && col2 >= d - kMixRope) {
            const int pr = (col2 - (d - kMixRope)) / 2;
            rope_pair(o0, o1, a.inv_cos[pr], a.inv_sin[pr], true);
        }
        const long long o = b * a.out_stride_b + static_cast<long long>(hh) * d + col2;
        if (a.out_bf16) {
            static_cast<uint16_t*>(a.out)[o] = f32_to_bf16(o0);
            static_cast<uint16_t*>(a.out)[o + 1] = f32_to_bf16(o1);
        } else {
            static_cast<float*>(a.out)[o] = o0;
            static_cast<float*>(a.out)[o + 1] = o1;
        }
    }
    if (a.lse && cb == 0 && lane == 0) a.lse[static_cast<long long>(b) * a.h + hh] = M + logf(den);
    // device counters: every reader of the state ran in the attention launch
    if (a.dev_adv && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) dev_advance(a.dev_adv, a.m, a.w, a.max_comp);
}

}  // namespace

int attn_dense_splits(int n_max) { return n_max > 0 ? (n_max + kDenseRows - 1) / kDenseRows : 1; }

hipError_t launch_attn_dense_bf16(AttnArgs a, const PrepArgs& prep, const void* x0, long long x0_stride_b,
                                  const void* x1, long long x1_stride_b, hipStream_t s) {
    if (a.d > kDenseMaxD || a.d % 32 != 0 || a.h % kHeadGroup != 0 || !x1) return hipErrorInvalidValue;
    const int ns = attn_dense_splits(a.n_max);
    if (ns > kWave) return hipErrorInvalidValue;
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
    const int att_wgs = groups * ns;
    // a long main block (main_wgs > 1), or any block with mixed KV, is
    // folded into the attention workgroups; otherwise one job workgroup
    // compresses it.  With mixed KV the entry goes to the workspace in
    // float32 and the merge packs it (its row scale spans every slice).
    const bool fold = prep.completes && (prep.main_wgs > 1 || a.kv_mixed);
    float* entry_f32 = a.kv_mixed && prep.completes ? a.ws_ml + static_cast<size_t>(a.batch) * a.h * ns * 2 : nullptr;
    uint8_t* rec0 = entry_f32 ? static_cast<uint8_t*>(prep.comp_kv) + static_cast<long long>(prep.n_comp) * kMixRec
                              : nullptr;
    const int prep_wgs = prep.completes && !fold ? 2 : 1;
    int fold_ch = 0;
    if (fold) {  // a power of two, so the slices of a channel merge by lane swaps
        fold_ch = kFoldMinCh;
        while (fold_ch * att_wgs < a.d) fold_ch *= 2;
    }
    const int extra = 1 + (x0 || entry_f32 ? 1 : 0);
    hipLaunchKernelGGL(k_attn_dense_bf16, dim3(att_wgs + prep_wgs, a.batch), dim3(kDenseThreads), lds, s, a, ns,
                       prep_wgs, prep, extra, fold_ch, entry_f32);
    const int col_blocks = (a.d + kMergeCols - 1) / kMergeCols;
    hipLaunchKernelGGL(k_attn_merge_rows, dim3(a.h * col_blocks, a.batch), dim3(kMergeThreads), 0, s, a, ns,
                       static_cast<const uint16_t*>(x0), x0_stride_b, static_cast<const uint16_t*>(x1), x1_stride_b,
                       entry_f32, rec0, prep.comp_kv_stride_b, prep.entry_cos, prep.entry_sin);
    return hipGetLastError();
}

}  // namespace csa

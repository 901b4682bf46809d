// Compressor reduce for one block of one sequence, run by one workgroup.
//
// Page 1, dsv4/kernels/cuda/compressor_reduce.cu (paper eq. 9-12), with the
// fix of pages 2/3: per channel, softmax over the block's rows of Z + B (the
// positional bias is added to the logits only), then the weighted sum of C.
// Optional weighted RMSNorm of the output row (apply_kv_norm_kernel).
//
// Threads stride over channels so every row read is coalesced.  The softmax
// runs in one pass with a running maximum (rescaling the partial sums when the
// maximum grows), so each row is read once.
#pragma once

#include "common.h"

namespace csa {

// z, c: this sequence's rows, pointing at the first row of block i (local
// index); global block g = first_block + i decides whether the overlapped
// form joins the previous block's a half.  ybuf: d floats of LDS (norm only);
// red: blockDim/64 floats of LDS.  keep (LDS, may be ybuf): if set, also
// receives the output as stored (after the bf16 rounding when out_bf16), and
// the workgroup is synchronised before the call returns.
__device__ inline void compress_block(const float* __restrict__ z, const float* __restrict__ c,
                                      const float* __restrict__ bias, const float* __restrict__ norm_w,
                                      void* __restrict__ out_row, bool out_bf16, int m, int d,
                                      bool overlap, long long g, float* ybuf, float* red,
                                      float* keep = nullptr, long long prev_off = 0) {
    const int width = overlap ? 2 * d : d;
    const bool joint = overlap && g > 0;  // previous block's a half joins the softmax
    const int own_col = overlap ? d : 0;  // this block's rows: b half when overlapped
    const int rows = joint ? 2 * m : m;   // logical rows of the joint softmax
    float ss = 0.f;
    for (int ch = threadIdx.x; ch < d; ch += blockDim.x) {
        // one pass with a running max; the rows' loads are issued in batches
        // so their latencies overlap
        float mx = -INFINITY, den = 0.f, acc = 0.f;
        constexpr int kBatch = 8;
        for (int r0 = 0; r0 < rows; r0 += kBatch) {
            float lz[kBatch], lc[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int r = r0 + u;
                lz[u] = -INFINITY;
                lc[u] = 0.f;
                if (r < rows) {
                    // logical row r: block g-1's a half first (rows before z), then own rows
                    const bool prev = joint && r < m;
                    const int t = prev ? r : (joint ? r - m : r);
                    const int col = prev ? ch : own_col + ch;
                    // the previous block's rows: just before z, or prev_off elements from it
                    const long long o = (prev ? (prev_off ? prev_off : -static_cast<long long>(m) * width) : 0) +
                                        static_cast<long long>(t) * width + col;
                    lz[u] = z[o] + bias[t * width + col];
                    lc[u] = c[o];
                }
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (r0 + u < rows) {
                    if (lz[u] > mx) {
                        const float sc = expf(mx - lz[u]);  // 0 on the first row
                        den *= sc;
                        acc *= sc;
                        mx = lz[u];
                    }
                    const float e = expf(lz[u] - mx);
                    den += e;
                    acc += e * lc[u];
                }
            }
        }
        const float y = acc / den;
        if (norm_w) {
            ybuf[ch] = y;
            ss += y * y;
        } else if (out_bf16) {
            const uint16_t yb = f32_to_bf16(y);
            static_cast<uint16_t*>(out_row)[ch] = yb;
            if (keep) keep[ch] = bf16_to_f32(yb);
        } else {
            static_cast<float*>(out_row)[ch] = y;
            if (keep) keep[ch] = y;
        }
    }
    if (!norm_w) {
        if (keep) __syncthreads();
        return;
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int wv = 0; wv < static_cast<int>(blockDim.x / kWave); ++wv) tot += red[wv];
    const float inv = 1.0f / sqrtf(tot / d + 1e-6f);
    for (int ch = threadIdx.x; ch < d; ch += blockDim.x) {
        const float y = ybuf[ch] * inv * norm_w[ch];
        if (out_bf16) {
            const uint16_t yb = f32_to_bf16(y);
            static_cast<uint16_t*>(out_row)[ch] = yb;
            if (keep) keep[ch] = bf16_to_f32(yb);
        } else {
            static_cast<float*>(out_row)[ch] = y;
            if (keep) keep[ch] = y;
        }
    }
    if (keep) __syncthreads();
}

// Long blocks (large m, no norm) split over workgroups and row slices: this
// workgroup computes channels [ch0, ch0 + nch) of the output row; its
// blockDim.x / nch thread slices each take a contiguous range of the m rows
// (all of a slice's loads in flight at once), and the slices' running
// (max, denominator, weighted sum) are combined in LDS:
// M = max_s mx_s, den = sum_s den_s e^(mx_s - M), acc likewise, y = acc / den.
// part: 3 * blockDim.x floats of LDS.  Plain (non-overlapped) blocks only.

// One row of a slice into its running (max, denominator, weighted sum).
__device__ inline void slice_row_update(float lz, float lc, float& mx, float& den, float& acc) {
    if (lz > mx) {
        const float sc = expf(mx - lz);  // 0 on the slice's first row
        den *= sc;
        acc *= sc;
        mx = lz;
    }
    const float e = expf(lz - mx);
    den += e;
    acc += e * lc;
}

// One lane-swap level of slice_merge: the running sums of slice partners
// O lanes apart combined (DPP moves, no LDS).
template <int O>
__device__ inline void slice_swap(float& m2, float& d2, float& a2) {
    const float mo = xor_lanes_f32<O>(m2);
    const float dn = xor_lanes_f32<O>(d2);
    const float ao = xor_lanes_f32<O>(a2);
    const float M = fmaxf(m2, mo);
    const float f1 = m2 == -INFINITY ? 0.f : expf(m2 - M);  // an empty slice adds nothing
    const float f2 = mo == -INFINITY ? 0.f : expf(mo - M);
    d2 = d2 * f1 + dn * f2;
    a2 = a2 * f1 + ao * f2;
    m2 = M;
}

// The slices' running sums combined in LDS; the output channels written.
__device__ inline void slice_merge(float mx, float den, float acc, void* __restrict__ out_row, bool out_bf16, int d,
                                   int ch0, int nch, float* part) {
    const int slices = blockDim.x / nch;
    const int t = threadIdx.x % nch;
    const int ch = ch0 + t;
    const int sl = threadIdx.x / nch;
    part[threadIdx.x] = mx;
    part[blockDim.x + threadIdx.x] = den;
    part[2 * blockDim.x + threadIdx.x] = acc;
    __syncthreads();
    if ((slices & (slices - 1)) == 0 && slices <= kWave && slices * nch == static_cast<int>(blockDim.x)) {
        // one thread per (channel, slice), a channel's slices in consecutive
        // lanes: the slices' (max, sum, weighted sum) merged by lane swaps
        const int tc = threadIdx.x / slices;
        const int s2 = threadIdx.x % slices;
        float m2 = part[s2 * nch + tc];
        float d2 = part[blockDim.x + s2 * nch + tc];
        float a2 = part[2 * blockDim.x + s2 * nch + tc];
        if (slices > 1) slice_swap<1>(m2, d2, a2);
        if (slices > 2) slice_swap<2>(m2, d2, a2);
        if (slices > 4) slice_swap<4>(m2, d2, a2);
        if (slices > 8) slice_swap<8>(m2, d2, a2);
        if (slices > 16) slice_swap<16>(m2, d2, a2);
        if (slices > 32) slice_swap<32>(m2, d2, a2);
        if (s2 == 0 && ch0 + tc < d) {
            const float y = a2 / d2;
            if (out_bf16)
                static_cast<uint16_t*>(out_row)[ch0 + tc] = f32_to_bf16(y);
            else
                static_cast<float*>(out_row)[ch0 + tc] = y;
        }
        return;
    }
    if (sl == 0 && ch < d) {
        float M = -INFINITY;
        for (int s2 = 0; s2 < slices; ++s2) M = fmaxf(M, part[s2 * nch + t]);
        float dsum = 0.f, asum = 0.f;
        for (int s2 = 0; s2 < slices; ++s2) {
            const float mxs = part[s2 * nch + t];
            if (mxs == -INFINITY) continue;  // an empty slice
            const float f = expf(mxs - M);
            dsum += part[blockDim.x + s2 * nch + t] * f;
            asum += part[2 * blockDim.x + s2 * nch + t] * f;
        }
        const float y = asum / dsum;
        if (out_bf16)
            static_cast<uint16_t*>(out_row)[ch] = f32_to_bf16(y);
        else
            static_cast<float*>(out_row)[ch] = y;
    }
}

// This thread's rows of the slice: [r_lo, r_hi) of channel ch (empty when
// the thread has no slice or channel).
__device__ inline void slice_rows(int m, int d, int ch0, int nch, int& ch, int& r_lo, int& r_hi) {
    const int slices = blockDim.x / nch;
    const int t = threadIdx.x % nch;
    const int sl = threadIdx.x / nch;
    ch = ch0 + t;
    const int per = (m + slices - 1) / slices;
    r_lo = sl * per;
    r_hi = min(m, r_lo + per);
    if (sl >= slices || ch >= d) r_hi = r_lo;
}

__device__ inline void compress_block_slice(const float* __restrict__ z, const float* __restrict__ c,
                                            const float* __restrict__ bias, void* __restrict__ out_row,
                                            bool out_bf16, int m, int d, int ch0, int nch, float* part) {
    int ch, r_lo, r_hi;
    slice_rows(m, d, ch0, nch, ch, r_lo, r_hi);
    float mx = -INFINITY, den = 0.f, acc = 0.f;
    constexpr int kBatch = 16;
    for (int r0 = r_lo; r0 < r_hi; r0 += kBatch) {
        float lz[kBatch], lc[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int r = r0 + u;
            lz[u] = -INFINITY;
            lc[u] = 0.f;
            if (r < r_hi) {
                const long long o = static_cast<long long>(r) * d + ch;
                lz[u] = z[o] + bias[o];
                lc[u] = c[o];
            }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (r0 + u < r_hi) slice_row_update(lz[u], lc[u], mx, den, acc);
    }
    slice_merge(mx, den, acc, out_row, out_bf16, d, ch0, nch, part);
}

}  // namespace csa

// Compressor reduce: one compressed entry per block of m token rows.
//
// Page 1, dsv4/kernels/cuda/compressor_reduce.cu (paper eq. 9-12), with the
// fix of pages 2/3: per channel, softmax over the block's rows of Z + B (the
// positional bias is added to the logits only), then the weighted sum of C.
// Optional weighted RMSNorm of each output row (apply_kv_norm_kernel).
//
// Work is tiny (a few KB per block); one workgroup per (block, sequence),
// threads stride over channels so every row read is coalesced.  The two
// passes (max, then exp-sum and weighted sum) run out of L1.
#include "common.h"
#include "kernels.h"

namespace csa {

namespace {

constexpr int kCompressThreads = 256;

__global__ __launch_bounds__(kCompressThreads) void k_compress(
    const float* __restrict__ z, const float* __restrict__ c, const float* __restrict__ bias,
    const float* __restrict__ norm_w, void* __restrict__ out, int out_bf16, int m, int d,
    int overlap, int first_block, long long zc_stride_b, long long out_stride_b) {
    extern __shared__ float ybuf[];  // [d], only used with norm_w
    __shared__ float red[kCompressThreads / kWave];
    const int i = blockIdx.x;
    const int b = blockIdx.y;
    const long long g = static_cast<long long>(first_block) + i;
    const int width = overlap ? 2 * d : d;
    const float* zb = z + b * zc_stride_b;
    const float* cb = c + b * zc_stride_b;
    const long long cur = static_cast<long long>(i) * m * width;   // first row of block i
    const long long prev = cur - static_cast<long long>(m) * width;  // block i-1 (may be < 0)
    const bool joint = overlap && g > 0;     // previous block's a half joins the softmax
    const int own_col = overlap ? d : 0;     // this block's rows: b half when overlapped

    float ss = 0.f;
    for (int ch = threadIdx.x; ch < d; ch += blockDim.x) {
        float mx = -INFINITY;
        if (joint) {
            for (int t = 0; t < m; ++t)
                mx = fmaxf(mx, zb[prev + (long long)t * width + ch] + bias[t * width + ch]);
        }
        for (int t = 0; t < m; ++t)
            mx = fmaxf(mx, zb[cur + (long long)t * width + own_col + ch] + bias[t * width + own_col + ch]);
        float den = 0.f, acc = 0.f;
        if (joint) {
            for (int t = 0; t < m; ++t) {
                const float e = expf(zb[prev + (long long)t * width + ch] + bias[t * width + ch] - mx);
                den += e;
                acc += e * cb[prev + (long long)t * width + ch];
            }
        }
        for (int t = 0; t < m; ++t) {
            const long long o = cur + (long long)t * width + own_col + ch;
            const float e = expf(zb[o] + bias[t * width + own_col + ch] - mx);
            den += e;
            acc += e * cb[o];
        }
        const float y = acc / den;
        if (norm_w) {
            ybuf[ch] = y;
            ss += y * y;
        } else if (out_bf16) {
            static_cast<uint16_t*>(out)[b * out_stride_b + (long long)i * d + ch] = f32_to_bf16(y);
        } else {
            static_cast<float*>(out)[b * out_stride_b + (long long)i * d + ch] = y;
        }
    }
    if (!norm_w) return;
    ss = wave_sum(ss);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int wv = 0; wv < static_cast<int>(blockDim.x / kWave); ++wv) tot += red[wv];
    const float inv = 1.0f / sqrtf(tot / d + 1e-6f);
    for (int ch = threadIdx.x; ch < d; ch += blockDim.x) {
        const float y = ybuf[ch] * inv * norm_w[ch];
        if (out_bf16)
            static_cast<uint16_t*>(out)[b * out_stride_b + (long long)i * d + ch] = f32_to_bf16(y);
        else
            static_cast<float*>(out)[b * out_stride_b + (long long)i * d + ch] = y;
    }
}

}  // namespace

hipError_t launch_compress(const float* z, const float* c, const float* bias, const float* norm_w,
                           void* out, bool out_bf16, int batch, int n_blocks, int m, int d,
                           bool overlap, int first_block, long long zc_stride_b,
                           long long out_stride_b, hipStream_t s) {
    if (n_blocks == 0) return hipSuccess;
    const int threads = d >= kCompressThreads ? kCompressThreads : ((d + kWave - 1) / kWave) * kWave;
    const size_t lds = norm_w ? sizeof(float) * d : 0;
    hipLaunchKernelGGL(k_compress, dim3(n_blocks, batch), dim3(threads), lds, s, z, c, bias, norm_w,
                       out, out_bf16 ? 1 : 0, m, d, overlap ? 1 : 0, first_block, zc_stride_b,
                       out_stride_b);
    return hipGetLastError();
}

}  // namespace csa

// Standalone compressor reduce: one workgroup per (block, sequence).  The
// arithmetic is compress_block (compress_impl.h).
#include "compress_impl.h"
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
    const int width = overlap ? 2 * d : d;
    const long long row0 = static_cast<long long>(i) * m * width;
    const int es = out_bf16 ? 2 : 4;
    char* orow = static_cast<char*>(out) + (b * out_stride_b + static_cast<long long>(i) * d) * es;
    compress_block(z + b * zc_stride_b + row0, c + b * zc_stride_b + row0, bias, norm_w, orow, out_bf16 != 0,
                   m, d, overlap != 0, static_cast<long long>(first_block) + i, ybuf, red);
}

}  // namespace

int compress_threads(int d) { return d >= kCompressThreads ? kCompressThreads : ((d + kWave - 1) / kWave) * kWave; }

hipError_t launch_compress(const float* z, const float* c, const float* bias, const float* norm_w,
                           void* out, bool out_bf16, int batch, int n_blocks, int m, int d,
                           bool overlap, int first_block, long long zc_stride_b,
                           long long out_stride_b, hipStream_t s) {
    if (n_blocks == 0) return hipSuccess;
    const size_t lds = norm_w ? sizeof(float) * d : 0;
    hipLaunchKernelGGL(k_compress, dim3(n_blocks, batch), dim3(compress_threads(d)), lds, s, z, c, bias, norm_w,
                       out, out_bf16 ? 1 : 0, m, d, overlap ? 1 : 0, first_block, zc_stride_b, out_stride_b);
    return hipGetLastError();
}

}  // namespace csa

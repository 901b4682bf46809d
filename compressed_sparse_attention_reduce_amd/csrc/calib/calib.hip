// Calibration probes (libcsa_calib.so, include/csa_calib.h), not a step of
// the method and not part of libcsa.so: a plain streaming read of a buffer
// (the practical HBM read ceiling that the memory-bound kernels are compared
// with: one launch reading each byte once, as the index scan reads its key
// cache) and the matrix cores' issue ceiling.
#include "csa_calib.h"

#include "../common.h"

namespace csa {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeInFlight = 4;  // 16-byte loads per thread per round (the fastest measured)

__global__ __launch_bounds__(kProbeThreads) void k_read_probe(const uint4* __restrict__ p, long long n16,
                                                              unsigned* __restrict__ sink) {
    const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
    long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kProbeInFlight - 1) * stride < n16; i += kProbeInFlight * stride) {
        uint4 v[kProbeInFlight];
#pragma unroll
        for (int u = 0; u < kProbeInFlight; ++u) v[u] = p[i + u * stride];
#pragma unroll
        for (int u = 0; u < kProbeInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;  // keeps the loads; practically never taken
}

// Matrix-core issue ceiling: every wave runs four independent chains of
// v_mfma_f32_16x16x32_bf16 (16,384 FLOP each) with kValu float FMAs on
// independent registers between consecutive MFMAs, the ratio of vector work
// to matrix work that a kernel's epilogue imposes.  Operands come from the
// thread index (nothing folds); the sums reach `sink` only on a value that
// practically never occurs, so no work is removed.
template <int kValu>
__global__ __launch_bounds__(kProbeThreads) void k_mfma_probe(float* __restrict__ sink, int iters) {
    const int t = threadIdx.x + blockIdx.x * blockDim.x;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = static_cast<__bf16>(static_cast<float>((t + e) & 7) * 0.125f);
        b[e] = static_cast<__bf16>(static_cast<float>((t * 3 + e) & 7) * 0.0625f);
    }
    f32x4 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    float x[4] = {static_cast<float>(t & 15), 1.f, 2.f, 3.f};
    const float y = 1.0000001f, z = static_cast<float>(t & 3) * 1e-7f;
#pragma unroll 1
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
#pragma unroll
            for (int v = 0; v < kValu; ++v) x[(c + v) & 3] = fmaf(x[(c + v) & 3], y, z);
        }
    }
    float s = x[0] + x[1] + x[2] + x[3];
#pragma unroll
    for (int c = 0; c < 4; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    if (s == 1234567.f) sink[0] = s;
}

}  // namespace

int cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return n;
}

hipError_t launch_mfma_probe(float* sink, int waves_per_simd, int iters, int valu_per_mfma, hipStream_t s) {
    const int cus = cu_count();
    if (cus <= 0) return hipErrorInvalidDevice;
    const dim3 grid(cus * waves_per_simd), block(kProbeThreads);
    switch (valu_per_mfma) {
        case 0: hipLaunchKernelGGL(k_mfma_probe<0>, grid, block, 0, s, sink, iters); break;
        case 1: hipLaunchKernelGGL(k_mfma_probe<1>, grid, block, 0, s, sink, iters); break;
        case 2: hipLaunchKernelGGL(k_mfma_probe<2>, grid, block, 0, s, sink, iters); break;
        case 3: hipLaunchKernelGGL(k_mfma_probe<3>, grid, block, 0, s, sink, iters); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_read_probe(const void* buf, long long bytes, unsigned* sink, hipStream_t s) {
    if (bytes < 16) return hipSuccess;
    const int cus = cu_count();
    if (cus <= 0) return hipErrorInvalidDevice;
    hipLaunchKernelGGL(k_read_probe, dim3(2 * cus), dim3(kProbeThreads), 0, s, static_cast<const uint4*>(buf),
                       bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace csa

extern "C" {

int csa_read_probe(const void* buf, long long bytes, unsigned* sink, csa_stream stream) {
    if (bytes < 0 || (bytes >= 16 && (!buf || !sink)) || (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
        return CSA_ERR_INVALID_ARG;
    return csa::launch_read_probe(buf, bytes, sink, static_cast<hipStream_t>(stream)) == hipSuccess ? CSA_OK
                                                                                                     : CSA_ERR_LAUNCH;
}

int csa_mfma_probe(float* sink, int waves_per_simd, int iters, int valu_per_mfma, csa_stream stream) {
    if (!sink || waves_per_simd < 1 || waves_per_simd > 8 || iters < 1 || iters > (1 << 24) || valu_per_mfma < 0 ||
        valu_per_mfma > 3)
        return CSA_ERR_INVALID_ARG;
    return csa::launch_mfma_probe(sink, waves_per_simd, iters, valu_per_mfma, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? CSA_OK
               : CSA_ERR_LAUNCH;
}

}  // extern "C"

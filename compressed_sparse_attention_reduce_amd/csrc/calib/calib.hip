// Calibration probes (libcsa_calib.so, include/csa_calib.h), not a step of
// the method and not part of libcsa.so: a plain streaming read of a buffer
// (the practical HBM read ceiling that the memory-bound kernels are compared
// with: one launch reading each byte once, as the index scan reads its key
// cache), the matrix cores' issue ceiling, the arrival time of one shared
// row behind every workgroup's own loads (as the scan's query arrives behind
// the key tiles), and the cost of handing data from every workgroup to the
// last one inside a launch (release fence, ticket, acquire fence).
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

// s_waitcnt immediate that waits until at most n vector loads are
// outstanding (vmcnt split over bits 3:0 and 15:14), the other counters free
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0f70; }

// Shared-row arrival behind a flood of loads: every workgroup loads the same
// 16 KB row (four 16-byte pieces per thread, as a scan workgroup loads its
// query), then kTiles rounds of four 16-byte loads of its own slice of buf
// (as a scan wave fills its ring), then waits for the row alone and then for
// everything.  stamps[4 wg ..] = (start, row arrived, all arrived) in
// wall-clock ticks (wave 0's view).
template <int kTiles>
__global__ __launch_bounds__(kProbeThreads) void k_queue_probe(const uint4* __restrict__ row,
                                                               const uint4* __restrict__ buf,
                                                               long long* __restrict__ stamps,
                                                               unsigned* __restrict__ sink) {
    const long long t0 = wall_clock64();
    uint4 q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] = row[threadIdx.x + u * kProbeThreads];
    __builtin_amdgcn_sched_barrier(0);
    constexpr int kLoads = kTiles * 4;
    uint4 k[kLoads > 0 ? kLoads : 1];
    const long long base = static_cast<long long>(blockIdx.x) * kProbeThreads * kLoads;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) k[i] = buf[base + static_cast<long long>(i) * kProbeThreads + threadIdx.x];
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoads));  // the row's loads are the oldest
    __builtin_amdgcn_sched_barrier(0);
    const long long t1 = wall_clock64();
    uint32_t acc = q[0].x ^ q[1].y ^ q[2].z ^ q[3].w;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) acc ^= k[i].x ^ k[i].w;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __builtin_amdgcn_sched_barrier(0);
    const long long t2 = wall_clock64();
    if (threadIdx.x == 0) {
        stamps[4 * static_cast<long long>(blockIdx.x) + 0] = t0;
        stamps[4 * static_cast<long long>(blockIdx.x) + 1] = t1;
        stamps[4 * static_cast<long long>(blockIdx.x) + 2] = t2;
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;  // keeps the loads; practically never taken
}

// Hand-off inside a launch: every workgroup writes 256 floats of its own;
// with kHandoff, after a workgroup barrier one thread makes them visible
// device-wide (a release fence) and takes a ticket, and the workgroup
// holding the last ticket reads every workgroup's floats after an acquire
// fence, writes 256 partial sums to out and resets the counter for the next
// launch (the usual last-workgroup reduction).
template <bool kHandoff>
__global__ __launch_bounds__(kProbeThreads) void k_handoff_probe(float* __restrict__ data, unsigned* counter,
                                                                 float* __restrict__ out) {
    __shared__ unsigned last;
    data[static_cast<long long>(blockIdx.x) * kProbeThreads + threadIdx.x] =
        static_cast<float>(blockIdx.x) + static_cast<float>(threadIdx.x) * 0.5f;
    if constexpr (kHandoff) {
        __syncthreads();
        if (threadIdx.x == 0) {
            __threadfence();
            last = atomicAdd(counter, 1u) == gridDim.x - 1 ? 1u : 0u;
        }
        __syncthreads();
        if (last == 0u) return;  // workgroup-uniform
        __threadfence();
        float sum = 0.f;
        for (long long i = threadIdx.x; i < static_cast<long long>(gridDim.x) * kProbeThreads; i += kProbeThreads)
            sum += data[i];
        out[threadIdx.x] = sum;
        if (threadIdx.x == 0) *counter = 0u;
    }
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

int queue_probe_workgroups() { return 2 * cu_count(); }

hipError_t launch_queue_probe(const void* row, const void* buf, int tiles, long long* stamps, unsigned* sink,
                              hipStream_t s) {
    const int wgs = queue_probe_workgroups();
    if (wgs <= 0) return hipErrorInvalidDevice;
    const uint4* r = static_cast<const uint4*>(row);
    const uint4* b = static_cast<const uint4*>(buf);
    switch (tiles) {
        case 0: hipLaunchKernelGGL(k_queue_probe<0>, dim3(wgs), dim3(kProbeThreads), 0, s, r, b, stamps, sink); break;
        case 2: hipLaunchKernelGGL(k_queue_probe<2>, dim3(wgs), dim3(kProbeThreads), 0, s, r, b, stamps, sink); break;
        case 4: hipLaunchKernelGGL(k_queue_probe<4>, dim3(wgs), dim3(kProbeThreads), 0, s, r, b, stamps, sink); break;
        case 8: hipLaunchKernelGGL(k_queue_probe<8>, dim3(wgs), dim3(kProbeThreads), 0, s, r, b, stamps, sink); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_handoff_probe(float* data, unsigned* counter, float* out, int wgs, bool handoff, hipStream_t s) {
    if (handoff)
        hipLaunchKernelGGL(k_handoff_probe<true>, dim3(wgs), dim3(kProbeThreads), 0, s, data, counter, out);
    else
        hipLaunchKernelGGL(k_handoff_probe<false>, dim3(wgs), dim3(kProbeThreads), 0, s, data, counter, out);
    return hipGetLastError();
}

}  // namespace csa

extern "C" {

int csa_probe_workgroups(void) { return csa::queue_probe_workgroups(); }

int csa_queue_probe(const void* row, const void* buf, long long buf_bytes, int tiles, long long* stamps,
                    long long n_stamps, unsigned* sink, csa_stream stream) {
    if (!row || !stamps || !sink || (tiles != 0 && tiles != 2 && tiles != 4 && tiles != 8) ||
        (reinterpret_cast<uintptr_t>(row) & 15) != 0 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0 ||
        (tiles > 0 && !buf))
        return CSA_ERR_INVALID_ARG;
    const long long wgs = csa::queue_probe_workgroups();
    if (wgs <= 0) return CSA_ERR_LAUNCH;
    if (n_stamps < 4 * wgs || (tiles > 0 && buf_bytes < wgs * csa::kProbeThreads * tiles * 4 * 16))
        return CSA_ERR_INVALID_ARG;
    return csa::launch_queue_probe(row, buf, tiles, stamps, sink, static_cast<hipStream_t>(stream)) == hipSuccess
               ? CSA_OK
               : CSA_ERR_LAUNCH;
}

int csa_handoff_probe(float* data, long long n_floats, unsigned* counter, float* out, int wgs, int handoff,
                      csa_stream stream) {
    if (!data || !counter || !out || wgs < 1 || wgs > 65535 || n_floats < static_cast<long long>(wgs) * 256)
        return CSA_ERR_INVALID_ARG;
    return csa::launch_handoff_probe(data, counter, out, wgs, handoff != 0, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? CSA_OK
               : CSA_ERR_LAUNCH;
}

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

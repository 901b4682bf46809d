// Packing of main-KV rows into mixed records (mixed_kv.h): one wave per row,
// the NoPE part quantised to E4M3 with its row scale, the RoPE part rounded
// to bfloat16 (rows taken as already rotated, as the pages' kv_roped).
#include "common.h"
#include "kernels.h"
#include "mixed_kv.h"

namespace csa {

namespace {

constexpr int kPackThreads = 256;
constexpr int kPackRowsPerWg = kPackThreads / kWave;

__global__ __launch_bounds__(kPackThreads) void k_pack_kv_mixed(const void* __restrict__ x, int x_bf16,
                                                                uint8_t* __restrict__ rec, long long rows) {
    const long long row = static_cast<long long>(blockIdx.x) * kPackRowsPerWg + threadIdx.x / kWave;
    if (row >= rows) return;  // wave-uniform
    const long long o = row * kMixD;
    if (x_bf16) {
        const uint16_t* xr = static_cast<const uint16_t*>(x) + o;
        wave_pack_mixed([&](int j) { return bf16_to_f32(xr[j]); }, rec + row * kMixRec, nullptr, nullptr);
    } else {
        const float* xr = static_cast<const float*>(x) + o;
        wave_pack_mixed([&](int j) { return xr[j]; }, rec + row * kMixRec, nullptr, nullptr);
    }
}

}  // namespace

hipError_t launch_pack_kv_mixed(const void* x, bool x_bf16, uint8_t* rec, long long rows, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    const long long wgs = (rows + kPackRowsPerWg - 1) / kPackRowsPerWg;
    hipLaunchKernelGGL(k_pack_kv_mixed, dim3(static_cast<unsigned>(wgs)), dim3(kPackThreads), 0, s, x,
                       x_bf16 ? 1 : 0, rec, rows);
    return hipGetLastError();
}

}  // namespace csa

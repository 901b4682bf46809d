// First kernel of the fused decode step: every small independent job of the
// step in one launch.  Roles by blockIdx.x, one workgroup per sequence each:
//   0  append the new token's KV row to the SWA ring (page 1, P2: slot swa_head);
//   1  compress the block the token completes into comp_kv[n_comp] (if any);
//   2  compress the indexer key of that block into idx_keys[n_comp] (if any).
#include "compress_impl.h"
#include "kernels.h"

namespace csa {

namespace {

constexpr int kPrepThreads = 256;

__global__ __launch_bounds__(kPrepThreads) void k_step_prep(PrepArgs a) {
    __shared__ float ybuf[kPrepMaxD];
    __shared__ float red[kPrepThreads / kWave];
    const int role = blockIdx.x;
    const int b = blockIdx.y;
    if (role == 0) {
        const char* src = static_cast<const char*>(a.kv_new) + b * a.kv_new_stride_b * a.es;
        char* dst = static_cast<char*>(a.swa) + (b * a.swa_stride_b + static_cast<long long>(a.swa_slot) * a.d) * a.es;
        for (int o = threadIdx.x * 16; o < a.d * a.es; o += kPrepThreads * 16)
            *reinterpret_cast<uint4*>(dst + o) = *reinterpret_cast<const uint4*>(src + o);
    } else {
        if (!a.completes) return;
        const bool main = role == 1;
        const int d = main ? a.d : a.d_i;
        const float* z = (main ? a.z_main : a.z_idx) + b * (main ? a.zc_main_stride_b : a.zc_idx_stride_b);
        const float* c = (main ? a.c_main : a.c_idx) + b * (main ? a.zc_main_stride_b : a.zc_idx_stride_b);
        char* out = static_cast<char*>(main ? a.comp_kv : a.idx_keys) +
                    (b * (main ? a.comp_kv_stride_b : a.idx_keys_stride_b) + static_cast<long long>(a.n_comp) * d) * a.es;
        compress_block(z, c, main ? a.main_bias : a.idx_bias, main ? a.main_norm : a.idx_norm, out, a.es == 2, a.m, d,
                       a.overlap != 0, a.block, ybuf, red);
    }
}

}  // namespace

hipError_t launch_step_prep(const PrepArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(k_step_prep, dim3(a.completes ? 3 : 1, a.batch), dim3(kPrepThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace csa

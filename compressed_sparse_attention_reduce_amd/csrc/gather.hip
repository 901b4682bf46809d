// Gather into the preallocated gather_buf (standalone entry point).
//
// Page 1 commit message C2 (one (top_k + window, hd) buffer filled by slice
// assignment, no concatenation on the hot path) and C3 (the ring may wrap);
// page 1, PERFORMANCE_AUDIT.md, P2 (slot (swa_head + i) % W).  Compressed
// rows come first, then the window oldest to newest.
//
// One wave copies one row with 16-byte lanes (a 1 KB bf16 row of hd 512 is
// exactly one wave-wide load and store).  Row sources are read from the
// device-side top-k indices; the host never sees them.
#include "common.h"
#include "kernels.h"

namespace csa {

namespace {

constexpr int kGatherThreads = 256;
constexpr int kRowsPerWg = kGatherThreads / kWave;

__global__ __launch_bounds__(kGatherThreads) void k_gather(
    const char* __restrict__ comp_kv, int n_comp, const int* __restrict__ idx,
    const int* __restrict__ count, int k, const char* __restrict__ swa, int swa_head, int swa_len,
    int w, char* __restrict__ buf, int* __restrict__ n_valid, int row_bytes, long long kv_stride_b,
    long long swa_stride_b, long long buf_stride_b) {
    const int b = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    const int j = blockIdx.x * kRowsPerWg + threadIdx.x / kWave;
    int cnt = count ? count[b] : k;
    cnt = cnt < 0 ? 0 : (cnt > k ? k : cnt);
    if (n_comp <= 0) cnt = 0;
    if (j == 0 && lane == 0 && n_valid) n_valid[b] = cnt + swa_len;
    const char* src;
    if (j < cnt) {
        int r = idx[static_cast<long long>(b) * k + j];
        r = r < 0 ? 0 : (r >= n_comp ? n_comp - 1 : r);
        src = comp_kv + b * kv_stride_b + static_cast<long long>(r) * row_bytes;
    } else if (j < cnt + swa_len) {
        int slot = (swa_head - swa_len + (j - cnt)) % w;
        if (slot < 0) slot += w;
        src = swa + b * swa_stride_b + static_cast<long long>(slot) * row_bytes;
    } else {
        return;
    }
    char* dst = buf + b * buf_stride_b + static_cast<long long>(j) * row_bytes;
    for (int o = lane * 16; o < row_bytes; o += kWave * 16)
        *reinterpret_cast<uint4*>(dst + o) = *reinterpret_cast<const uint4*>(src + o);
}

}  // namespace

hipError_t launch_gather(const void* comp_kv, int n_comp, const int* idx, const int* count, int k,
                         const void* swa, int swa_head, int swa_len, int w, void* buf,
                         int* n_valid, int elem_bytes, int batch, int d, long long kv_stride_b,
                         long long swa_stride_b, long long buf_stride_b, hipStream_t s) {
    const int rows = k + swa_len;
    const int wgs = rows > 0 ? (rows + kRowsPerWg - 1) / kRowsPerWg : 1;
    hipLaunchKernelGGL(k_gather, dim3(wgs, batch), dim3(kGatherThreads), 0, s,
                       static_cast<const char*>(comp_kv), n_comp, idx, count, k,
                       static_cast<const char*>(swa), swa_head, swa_len, w, static_cast<char*>(buf),
                       n_valid, d * elem_bytes, kv_stride_b * elem_bytes, swa_stride_b * elem_bytes,
                       buf_stride_b * elem_bytes);
    return hipGetLastError();
}

}  // namespace csa

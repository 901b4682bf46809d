// Host-side launchers of the CSA kernels.  Arguments are validated by the
// C ABI layer (capi.hip) before any of these is called; launchers only size
// grids and enqueue work on `s`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa {

int device_cu_count();

// ---- compressor reduce -------------------------------------------------------
hipError_t launch_compress(const float* z, const float* c, const float* bias, const float* norm_w,
                           void* out, bool out_bf16, int batch, int n_blocks, int m, int d,
                           bool overlap, int first_block, long long zc_stride_b,
                           long long out_stride_b, hipStream_t s);

// ---- lightning-indexer score -------------------------------------------------
struct ScoreArgs {
    const void* q;
    const float* w;
    const void* k;
    float* scores;
    int batch, t, h_i, d_i, n;
    const int* q_pos;
    int ratio;
    long long q_stride_b, w_stride_b, k_stride_b, s_stride_b, ld_s;
    uint32_t* hist;  // optional [batch*t][kHistBins] radix histogram of the scores
};
hipError_t launch_index_score_bf16(const ScoreArgs& a, hipStream_t s);
hipError_t launch_index_score_f32(const ScoreArgs& a, hipStream_t s);

// ---- top-k -------------------------------------------------------------------
constexpr int kTopkMaxK = 2048;
constexpr int kHistBits = 12;               // first radix digit (from the score kernel)
constexpr int kHistBins = 1 << kHistBits;
size_t topk_workspace_bytes(int rows, int n, int k);
struct TopkArgs {
    const float* scores;
    int batch, t, n;
    long long ld_s, s_stride_b;
    int k;
    int* idx;
    int* count;
    void* ws;
};
// hist_ready: the workspace histogram was already filled by the score kernel
// (and zeroed before it); otherwise the launcher builds it.
hipError_t launch_topk(const TopkArgs& a, bool hist_ready, hipStream_t s);
// Zeroes the workspace histogram/counters so a score kernel can fill it.
hipError_t launch_topk_ws_clear(void* ws, int rows, int n, int k, hipStream_t s);
uint32_t* topk_ws_hist(void* ws);

// ---- gather ------------------------------------------------------------------
hipError_t launch_gather(const void* comp_kv, int n_comp, const int* idx, const int* count, int k,
                         const void* swa, int swa_head, int swa_len, int w, void* buf,
                         int* n_valid, int elem_bytes, int batch, int d, long long kv_stride_b,
                         long long swa_stride_b, long long buf_stride_b, hipStream_t s);

// ---- sparse attention ----------------------------------------------------------
size_t attn_workspace_bytes(bool bf16, int batch, int h, int d, int n_max);
hipError_t launch_attn_bf16(const void* q, const void* kv, const int* n_valid, const float* sink,
                            float scale, void* out, bool out_bf16, float* lse, int batch, int h,
                            int d, int n_max, long long q_stride_b, long long kv_stride_b,
                            long long out_stride_b, void* ws, hipStream_t s);
hipError_t launch_attn_f32(const void* q, const void* kv, const int* n_valid, const float* sink,
                           float scale, void* out, bool out_bf16, float* lse, int batch, int h,
                           int d, int n_max, long long q_stride_b, long long kv_stride_b,
                           long long out_stride_b, hipStream_t s);

// ---- small helpers for the fused step ------------------------------------------
hipError_t launch_swa_append(const void* kv_new, void* swa, int slot, int elem_bytes, int batch,
                             int d, long long kv_new_stride_b, long long swa_stride_b,
                             hipStream_t s);

}  // namespace csa

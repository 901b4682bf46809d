// Host-side launchers of the prefill-shaped kernels: many query tokens at
// consecutive positions against one compressed history.  Arguments are
// validated by the C ABI layer (capi.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kernels.h"

namespace csa {

// ---- multi-query index score + top-k -----------------------------------------
constexpr int kPrefillChunkRows = 256;  // query rows whose scores are held at once
struct IndexTopkArgs {
    const uint16_t* q;  // [t][64][128] bf16
    const float* w;     // [t][64] (E4M3: query scales folded in)
    const uint16_t* k;  // [n][128] bf16
    int t, n;
    long long pos0;     // position of query 0; < 0: no causal mask
    int ratio;
    int top_k;
    int* idx;           // [t][top_k]
    int* count;         // [t] or nullptr
    void* ws;
    // E4M3 queries and keys instead (k_scale != nullptr): q8 [t][64][128],
    // k8 [n][128] codes, k_scale [n] row scales; q and k unused then
    const uint8_t* q8;
    const uint8_t* k8;
    const float* k_scale;
    // with k_fp4: k8 [n][64] packed E2M1 codes, k_scale four E8M0 bytes per
    // key (one 32-bit word each)
    int k_fp4;
};
size_t index_topk_workspace_bytes(int t, int n, int top_k);
hipError_t launch_index_topk(const IndexTopkArgs& a, hipStream_t s);

// The multi-query bf16 scan on its own (h_i = 64, d_i = 128; a.cands unused):
// a.scores[b][row][key] for every row of every sequence.  Causal mask from
// a.q_pos when given, else position pos0 + row when pos0 >= 0, else none.
// Same bits as launch_index_score_bf16 for the same (query, key).
constexpr int kMqMinRows = 16;  // query rows per sequence from which it is used
hipError_t launch_index_score_mq(const ScoreArgs& a, long long pos0, hipStream_t s);
// The same over E4M3 queries and keys (h_i = 64, d_i = 128; a.cands unused).
hipError_t launch_index_score_mq_fp8(const Fp8ScoreArgs& a, long long pos0, hipStream_t s);

// ---- per-query sparse attention over indexed rows + the sliding window --------
struct PrefillAttnArgs {
    const uint16_t* q;        // [t][h][d]
    const uint16_t* comp_kv;  // [n_comp][d]
    int n_comp;
    const int* idx;           // [t][k]
    const int* count;         // [t] (nullptr: k)
    int k;
    const uint16_t* win_kv;   // [t + window - 1][d], row r = position pos0 - window + 1 + r
    int window;
    long long pos0;
    const float* sink;        // [h] or nullptr
    float scale;
    void* out;                // [t][h][d]
    bool out_bf16;
    float* lse;               // [t][h] or nullptr
    int t, h, d;
    // mixed main KV (d = 512): comp_kv and win_kv hold 592-byte records
    // (mixed_kv.h), and out's RoPE dims are rotated back at each query's
    // position with rows pos0 + r of the tables (kMixRope / 2 values a row)
    bool kv_mixed;
    const float* inv_cos;
    const float* inv_sin;
};
bool prefill_attn_supported(int h, int d);
hipError_t launch_prefill_attn(const PrefillAttnArgs& a, hipStream_t s);

}  // namespace csa

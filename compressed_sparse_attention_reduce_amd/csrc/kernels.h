// Host-side launchers of the CSA kernels.  Arguments are validated by the
// C ABI layer (capi.hip) before any of these is called; launchers only size
// grids and enqueue work on `s`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa {

int device_cu_count();

// calibration read (calib.hip): every 16-byte piece of buf read once

constexpr int kTopkMaxK = 2048;

// ---- compressor reduce -------------------------------------------------------
hipError_t launch_compress(const float* z, const float* c, const float* bias, const float* norm_w,
                           void* out, bool out_bf16, int batch, int n_blocks, int m, int d,
                           bool overlap, int first_block, long long zc_stride_b,
                           long long out_stride_b, hipStream_t s);

// ---- top-k candidates ------------------------------------------------------------
constexpr int kMaxCandM1 = 64;  // longest per-slot candidate list
// Per-slot candidate lists: [rows][slots][m + 1] composites: up to m of the
// slot's largest (zero padded), then a bound at least as large as every
// composite of the slot not listed.  Each wave of a producing workgroup
// extracts its mw largest (mw <= m) before the workgroup merges them.
struct CandArgs {
    unsigned long long* lists;
    int slots;
    int m;
    int mw;
    // Which keys a slot lists (0: not stated): slot s < stride / run holds the
    // keys whose position modulo stride lies in [s * run, (s + 1) * run); any
    // slots past those list single keys in full (bound 0).
    int run;
    int stride;
};
// m for slots of keys_per_slot keys (also mw, for a wave's share of them),
// or -1 if lists would be too long.
int topk_cand_m(int n, int k, int keys_per_slot);

// ---- counters of a decode step held on the device (graph replay) --------------
// Same layout as csa_dev_state.  A step reads them when its kernels run and
// k_step_advance moves them past the step afterwards.
struct DevState {
    int pos, n_comp, swa_head, swa_len, flags;
};
constexpr int kDevFlagCacheFull = 1;  // a completed block found the compressed cache full
// The counters as the kernels use them: every index kept inside the caches
// whatever the caller stored (pos >= 0, 0 <= n_comp <= max_comp, the ring
// head and length inside the window w).
__host__ __device__ inline DevState dev_load(const DevState* p, int w, int max_comp) {
    DevState s = *p;
    s.pos = s.pos < 0 ? 0 : s.pos;
    s.n_comp = s.n_comp < 0 ? 0 : (s.n_comp > max_comp ? max_comp : s.n_comp);
    s.swa_head = ((s.swa_head % w) + w) % w;
    s.swa_len = s.swa_len < 0 ? 0 : (s.swa_len > w ? w : s.swa_len);
    return s;
}
// The step completes a block (and has room for its entry).
__host__ __device__ inline bool dev_completes(const DevState& s, int m, int max_comp) {
    return s.pos % m == m - 1 && s.n_comp < max_comp;
}
// Move the counters past the step that read them (one thread, after every
// reader of this step is done).
// Entries a step scores and selects from: those before it plus the block it completes.
__host__ __device__ inline int dev_step_entries(const DevState& s, int m, int max_comp) {
    return s.n_comp + (dev_completes(s, m, max_comp) ? 1 : 0);
}
__host__ __device__ inline void dev_advance(DevState* st, int m, int w, int max_comp) {
    DevState s = dev_load(st, w, max_comp);
    if (s.pos % m == m - 1) {
        if (s.n_comp < max_comp) s.n_comp += 1;
        else s.flags |= kDevFlagCacheFull;
    }
    s.pos += 1;
    s.swa_head = (s.swa_head + 1) % w;
    s.swa_len = s.swa_len + 1 < w ? s.swa_len + 1 : w;
    *st = s;
}

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
    // optional top-k candidates: every workgroup writes the top m + 1 of its
    // keys to its slot of cands.lists (cands.slots must equal its grid width)
    CandArgs cands;
    // decode step with device counters: n = dev->n_comp when the kernel runs
    // (the grid is sized for the n given here, the cache capacity)
    const DevState* dev;
};
constexpr int kScoreWavesPerWg = 4;  // waves per workgroup of the bf16 score kernel
// Scan workgroups per row and keys per scan workgroup of the bf16 score
// kernel (extra = workgroups per row the kernel also runs for other jobs).
int index_score_bf16_wgs(int rows, int n, int extra);
int index_score_bf16_keys_per_wg(int rows, int n, int extra);
struct PrepArgs;
// fold (optional, one query row per sequence): the decode step's small jobs
// (step_prep.h) run by the first workgroups of each row; with fold->completes
// the kernel also scores the new key at index a.n (its indexer key is the
// one role 2 compresses) and gives it the last candidate slot.  a.n counts
// the keys already in the cache.
hipError_t launch_index_score_bf16(const ScoreArgs& a, const PrepArgs* fold, hipStream_t s);
hipError_t launch_index_score_f32(const ScoreArgs& a, hipStream_t s);

// ---- FP8 E4M3 indexer keys ------------------------------------------------------
// w_in / w_out non-null: the rows are a query's head rows and w_out[r] =
// w_in[r] * scale_r replaces scales[r] (the scale folded into the weight)
hipError_t launch_quantize_fp8(const void* x, bool x_bf16, uint8_t* codes, float* scales, long long rows, int d,
                               hipStream_t s, const float* w_in = nullptr, float* w_out = nullptr);
// FP4 E2M1 rows with one E8M0 scale per 32 elements (d a multiple of 32):
// packed codes [rows][d / 2], scales [rows][d / 32]
hipError_t launch_quantize_fp4(const void* x, bool x_bf16, uint8_t* codes, uint8_t* scales, long long rows, int d,
                               hipStream_t s);
struct Fp8ScoreArgs {
    const uint8_t* q;      // [B][t][64][128] E4M3
    const float* w;        // [B][t][64], query scales folded in (unless q_raw)
    const uint8_t* k;      // [B][n][128] E4M3
    const float* k_scale;  // [B][n]
    float* scores;
    int batch, t, n;
    const int* q_pos;
    int ratio;
    long long q_stride_b, w_stride_b, k_stride_b, ks_stride_b, s_stride_b, ld_s;
    // optional top-k candidates, as in ScoreArgs
    CandArgs cands;
    // decode step with device counters, as in ScoreArgs
    const DevState* dev;
    // non-null (decode step, t = 1): the query as bfloat16 [B][t][64][128]
    // (stride in elements) instead of q; every workgroup quantises each head
    // row as csa_quantize_fp8 does and multiplies w by the row's scale
    const uint16_t* q_raw;
    long long q_raw_stride_b;
    // non-zero: FP4 keys — k holds packed E2M1 rows (element 2j in the low
    // nibble of byte j of the 64-byte row, stride k_stride_b bytes) and
    // k_scale 32-bit words, byte j the E8M0 scale of elements 32 j .. 32 j +
    // 31 (stride ks_stride_b words)
    int k_fp4;
};
// Scan workgroups per row and keys per scan workgroup of the FP8 scan.
int index_score_fp8_wgs(int rows, int n, int extra);
int index_score_fp8_keys_per_wg(int rows, int n, int extra);
// fold: as for launch_index_score_bf16 (one query row per sequence); role 2
// quantises the new key (fold->idx_fp8) and scores it.
hipError_t launch_index_score_fp8(const Fp8ScoreArgs& a, const PrepArgs* fold, hipStream_t s);

// ---- top-k -------------------------------------------------------------------
size_t topk_workspace_bytes(int rows, int n, int k);
struct TopkArgs {
    const float* scores;
    int batch, t, n;
    long long ld_s, s_stride_b;
    int k;
    int* idx;
    int* count;
    void* ws;
    // decode step with device counters (one query row per sequence): n is
    // the state's entry count after the step's own block, not the field above
    const DevState* dev;
    int w, m, max_comp;
};
// cands: per-slot candidate lists already produced (by the score kernel), or
// nullptr (the launcher produces them itself when the rows are long).
hipError_t launch_topk(const TopkArgs& a, const CandArgs* cands, hipStream_t s);
// Many rows of at most 65536 scores: one workgroup per row, the row held in
// registers (no workspace); longer rows go to launch_topk.
hipError_t launch_topk_rows(const TopkArgs& a, hipStream_t s);

// ---- gather ------------------------------------------------------------------
hipError_t launch_gather(const void* comp_kv, int n_comp, const int* idx, const int* count, int k,
                         const void* swa, int swa_head, int swa_len, int w, void* buf,
                         int* n_valid, int elem_bytes, int batch, int d, long long kv_stride_b,
                         long long swa_stride_b, long long buf_stride_b, hipStream_t s);

// ---- mixed main-KV records (layout in mixed_kv.h) ---------------------------------
constexpr int kMixD = 512;        // row width
constexpr int kMixRope = 64;      // trailing RoPE dims, kept in bfloat16
constexpr int kMixNope = kMixD - kMixRope;
constexpr int kMixRec = 592;      // bytes per record: codes, RoPE, scale, pad
constexpr int kMixScaleOff = 576;
hipError_t launch_pack_kv_mixed(const void* x, bool x_bf16, uint8_t* rec, long long rows, hipStream_t s);

// ---- sparse attention ----------------------------------------------------------
struct AttnArgs {
    const uint16_t* q;
    long long q_stride_b;
    // plain mode: rows kv[b][0 .. n_valid[b]) of [batch][n_max][d]
    const uint16_t* kv;
    long long kv_stride_b;
    const int* n_valid;
    // gather mode (idx != nullptr): rows = comp_kv[idx[b][0 .. count[b])] then
    // the live SWA window; written to gather_buf and n_valid_out on the way.
    // dense mode (dense, idx == nullptr): rows = comp_kv[0 .. n_comp) then the
    // live SWA window (the HCA layers' attention)
    bool dense;
    const uint16_t* comp_kv;
    long long comp_kv_stride_b;
    int n_comp;
    const int* idx;
    const int* count;
    int k;
    const uint16_t* swa;
    long long swa_stride_b;
    int swa_head, swa_len, w;
    uint16_t* gather_buf;
    long long buf_stride_b;
    int* n_valid_out;
    // common
    const float* sink;
    float scale;
    void* out;
    bool out_bf16;
    float* lse;
    long long out_stride_b;
    int batch, h, d, n_max;
    void* ws;
    float* ws_o;   // set by the launcher
    float* ws_ml;  // set by the launcher
    // mixed main KV (mixed_kv.h): comp_kv, swa and gather_buf hold 592-byte
    // records (their strides in bytes; d = 512), decoded to bfloat16 on load;
    // inv_cos / inv_sin (nullable): the table row of the token's position,
    // the output's RoPE dims rotated back with it
    bool kv_mixed;
    const float* inv_cos;
    const float* inv_sin;
    // decode step with device counters (gather mode): n_comp, swa_head,
    // swa_len and the top-k row length are taken from dev when the kernel
    // runs, as the step after the prep jobs sees them (m, max_comp decide a
    // completed block); with mixed KV the inverse-RoPE row is rope_cos /
    // rope_sin + pos * kMixRope / 2
    const DevState* dev;
    int m, max_comp;
    const float* rope_cos;
    const float* rope_sin;
    int rope_rows;  // positions past the table use its last row
    // the fused top-k attention stores the step's position here for the
    // merge, which then advances *dev_adv (so no reader of the counters runs
    // after the advance within the step)
    int* dev_pos;
    DevState* dev_adv;
    // HCA step with device counters: the entry RoPE tables by block index
    // (mixed KV; blocks past the table use its last row); dev_pos then holds
    // (pos, n_comp, completes) as the attention launch saw them
    const float* comp_rope_cos;
    const float* comp_rope_sin;
    int comp_rope_rows;
};
size_t attn_workspace_bytes(bool bf16, int batch, int h, int d, int n_max);
int attn_max_splits();
int attn_max_rows();
hipError_t launch_attn_bf16(AttnArgs a, hipStream_t s);
// merge of the split partials already in a.ws (ws_o / ws_ml set), ns splits
hipError_t launch_attn_merge(const AttnArgs& a, int ns, hipStream_t s);
// The HCA step's attention (dense mode, a.dense): the rows before the step
// (a.n_comp entries, a.swa_len window rows ending at slot a.swa_head - 1) in
// 128-row splits, the step's jobs (prep) in the same launch, then a merge
// that adds the new rows x0 (the entry of a completed block, or nullptr)
// and x1 (the new token's row).  At most 64 splits.  Workspace:
// sizeof(float) * batch * h * attn_dense_splits(n_max) * (d + 2).
struct PrepArgs;
int attn_dense_splits(int n_max);
hipError_t launch_attn_dense_bf16(AttnArgs a, const PrepArgs& prep, const void* x0, long long x0_stride_b,
                                  const void* x1, long long x1_stride_b, hipStream_t s);
// The two-stage E4M3 selection (decode step, one query row per sequence):
// the k_cand best by E4M3 score (t.k = k_cand; from cands when given, else
// the exact path over t.scores), their exact scores from the bfloat16 keys
// and query (the bfloat16 scan's arithmetic), written as one candidate list
// per sequence: out[b][0 .. k_cand) composites (zero padded) and out[b][k_cand]
// = 0, for launch_topk_attn / launch_topk with CandArgs{out, 1, k_cand, k_cand}.
struct RescoreArgs {
    const uint16_t* q;      // [B][64][128] bfloat16
    long long q_stride_b;
    const float* w;         // [B][64]
    long long w_stride_b;
    const uint16_t* keys;   // [B][max_comp][128] bfloat16
    long long keys_stride_b;
    int n;                  // keys in the cache (indices are clamped below it)
    unsigned long long* out;
};
hipError_t launch_fp8_rescore(const TopkArgs& t, const CandArgs* cands, const RescoreArgs& r, hipStream_t s);
// The second stage for many query rows (a prefill chunk): row r's candidates
// cand[r][0 .. cand_count[r]) (kc a row), their exact scores from the
// bfloat16 row q[r] (64 x 128), w[r] (64) and keys [n][128], the k best of
// them sorted into idx[r] (-1 past the count) and count[r] (nullable).
struct RescoreRowsArgs {
    const uint16_t* q;
    const float* w;
    const uint16_t* keys;
    int n;
    const int* cand;
    const int* cand_count;
    int kc;
    int t, k;
    int* idx;
    int* count;
};
hipError_t launch_rescore_rows(const RescoreRowsArgs& a, hipStream_t s);
// decode step, bf16 gather mode, one query row per sequence: every attention
// workgroup selects the top k itself (from cands when given, else the
// exact path over the scores), then attends; topk idx / count written too.
hipError_t launch_topk_attn(const TopkArgs& t, const CandArgs* cands, AttnArgs a, hipStream_t s);
// workgroups launch_topk_attn starts (one 1024-thread workgroup per compute unit fits)
int topk_attn_workgroups(int batch, int h, int n_max);
hipError_t launch_attn_f32(const void* q, const void* kv, const int* n_valid, const float* sink,
                           float scale, void* out, bool out_bf16, float* lse, int batch, int h,
                           int d, int n_max, long long q_stride_b, long long kv_stride_b,
                           long long out_stride_b, hipStream_t s);

// ---- first kernel of the fused decode step ------------------------------------------
constexpr int kPrepMaxD = 4096;
struct PrepArgs {
    int batch, es, d, d_i, m, overlap, completes, n_comp;
    int main_wgs;  // > 1: the main block is compressed in that many channel slices (roles 1 .. main_wgs)
    int idx_fp8;   // the indexer keys are E4M3 codes with per-row scales (role 2 quantises the new key)
    int idx_fp4;   // the indexer keys are packed E2M1 codes, idx_scales 32-bit words of four E8M0
                   // block scales (role 2 quantises the new key; idx_fp8 is set too)
    float* idx_scales;
    long long idx_scales_stride_b;
    uint16_t* idx_keys_exact;  // E4M3 keys: also the bfloat16 key here (nullable)
    long long idx_keys_exact_stride_b;
    long long block;
    const void* kv_new;
    long long kv_new_stride_b;
    void* swa;
    long long swa_stride_b;
    int swa_slot;
    const float *z_main, *c_main, *z_idx, *c_idx;
    long long zc_main_stride_b, zc_idx_stride_b;
    const float *main_bias, *idx_bias, *main_norm, *idx_norm;
    void* comp_kv;
    long long comp_kv_stride_b;
    void* idx_keys;
    long long idx_keys_stride_b;
    // mixed main KV (mixed_kv.h; swa and comp_kv records, strides in bytes):
    // role 0 packs kv_new, role 1 packs the compressed entry with its RoPE
    // dims rotated by the table row entry_cos / entry_sin
    int kv_mixed;
    const float* entry_cos;
    const float* entry_sin;
    // device counters (nullptr: the host values above): completes, n_comp,
    // block and swa_slot come from dev; the block's Z/C rows are kept in a
    // ring of two blocks per array (dev_ring: [B][4][2m][width] floats, the
    // arrays z_main, c_main, z_idx, c_idx; z_* / c_* above are then the new
    // token's rows); comp_rope_cos / _sin: table bases (mixed KV)
    const DevState* dev;
    int max_comp;
    int swa_w;  // window rows (the ring head is kept below it)
    float* dev_ring;
    long long ring_stride_b;
    const float* comp_rope_cos;
    const float* comp_rope_sin;
    int comp_rope_rows;  // blocks past the table use its last row
};
hipError_t launch_step_prep(const PrepArgs& a, hipStream_t s);

}  // namespace csa

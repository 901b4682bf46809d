/*
 * csa.h — C ABI of the compressed-sparse-attention (CSA) decode path for
 * AMD Instinct MI355X (gfx950).
 *
 * Five steps and their fused composition, as described on the source pages
 * (git compare views of the nvfp4-megamoe-kernel repository, a DeepSeek-V4
 * inference bring-up):
 *
 *   1. csa_compress     — compressor reduce: per channel, softmax over a block's
 *                         token rows of Z + B, then the weighted sum of C.
 *   2. csa_index_score  — lightning indexer: sum over heads of w * ReLU(q . K),
 *                         one key per compressed block shared by every head.
 *   3. csa_topk         — fixed-shape top-k, score descending, lower index first.
 *   4. csa_gather       — selected compressed rows, then the sliding window,
 *                         into one preallocated gather_buf.
 *   5. csa_sparse_attn  — one softmax over gather_buf rows (K = V) plus a
 *                         per-head sink logit that adds to the denominator only.
 *   6. csa_decode_step  — 1..5 for one new token of one layer, stream-ordered.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.   Every tensor argument is DEVICE memory owned by the caller; the
 *           library allocates nothing, frees nothing and keeps no state
 *           between calls other than the thread-local error message and a
 *           cache of each device's compute-unit count.
 *           Scratch memory is passed in as a workspace whose size is queried
 *           first (the *_workspace_size functions).
 * Layout.   Row-major.  "[B][N][D] with stride_b" means element (b, n, d)
 *           lives at base + b * stride_b + n * D + d, counted in ELEMENTS of
 *           the tensor's own type.  Batch strides may be 0 only where stated.
 * Types.    csa_dtype selects float32 or bfloat16 storage for the tensors an
 *           entry point documents as "dtype"; everything else is float32
 *           (weights, biases, sinks, scores) or int32 (indices, counts).
 *           Arithmetic is float32 throughout; bfloat16 outputs are rounded
 *           once, to nearest even.
 * Streams.  All work is enqueued on `stream` (a hipStream_t; NULL = the
 *           default stream).  No call synchronises the host, reads device
 *           memory on the host, or allocates; every call can be recorded
 *           into a HIP graph.
 * Errors.   Only host-known integers and pointers are validated.  A failed
 *           check returns CSA_ERR_INVALID_ARG (or CSA_ERR_UNSUPPORTED /
 *           CSA_ERR_WORKSPACE) before anything is enqueued; a launch failure
 *           returns CSA_ERR_LAUNCH.  csa_last_error() describes the last
 *           non-OK status of the calling thread.  Device-side index values
 *           are clamped into range, never trusted for memory addressing.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CSA_OK = 0,
    CSA_ERR_INVALID_ARG = -1,
    CSA_ERR_UNSUPPORTED = -2,
    CSA_ERR_LAUNCH = -3,
    CSA_ERR_WORKSPACE = -4
} csa_status;

/* CSA_FP8_E4M3 (OCP E4M3 codes, one byte per element) and CSA_FP4_E2M1
 * (E2M1 codes, two per byte, with E8M0 block scales: section 2d) are
 * accepted only where an entry point says so. */
typedef enum { CSA_F32 = 0, CSA_BF16 = 1, CSA_FP8_E4M3 = 2, CSA_FP4_E2M1 = 3 } csa_dtype;

typedef void *csa_stream; /* hipStream_t */

/* Message for the calling thread's last non-OK status ("" if none). */
const char *csa_last_error(void);

/* ------------------------------------------------------------------------
 * 1. Compressor reduce.
 *
 * Source: page 1 (compare v0.1-e2e-working...v-c1-c2-c3-20260602), file
 * dsv4/kernels/cuda/compressor_reduce.cu, header (paper eq. 9-12) and the
 * kernels hca_compress_reduce_kernel / csa_compress_reduce_kernel, with the
 * fix of page 2 and page 3 ("Fix two correctness bugs: compressor pos bias on
 * KV"): B is added to the logits Z only, never to C.  Optional weighted
 * RMSNorm of each output row (apply_kv_norm_kernel, eps 1e-6).
 *
 * overlap = 0: block i of batch b uses rows i*m .. i*m+m-1 of Z and C
 *   ([B][rows][d], stride_b = zc_stride_b floats) with bias row t for its t-th
 *   row; B is [m][d].
 * overlap = 1: Z, C rows are 2*d wide (a half | b half) and B is [m][2*d].
 *   Global block g = first_block + i uses, in one joint softmax, the m rows of
 *   block g-1 from the a half followed by its own m rows from the b half; block
 *   g = 0 uses its own b-half rows only.  z and c point at the first row of
 *   block first_block; when first_block > 0 the m rows before z and c (block
 *   first_block - 1) must be readable.
 * out:    [B][n_blocks][d] of out_dtype, stride_b = out_stride_b elements.
 * norm_w: [d] float32 or NULL (no norm).
 * Limits: 1 <= m <= 1024, 1 <= d <= 4096, batch >= 1, n_blocks >= 0.
 * ------------------------------------------------------------------------ */
int csa_compress(const float *z, const float *c, const float *bias, const float *norm_w,
                 void *out, csa_dtype out_dtype, int batch, int n_blocks, int m, int d,
                 int overlap, int first_block, long long zc_stride_b, long long out_stride_b,
                 csa_stream stream);

/* ------------------------------------------------------------------------
 * 2. Lightning-indexer score.
 *
 * Source: page 1, ARCHITECTURE_AND_MEMORY_AUDIT.md, finding F3 (paper
 * section 2.3.1, eq. 16): I[t,s] = sum_h w[t,h] * ReLU(q[t,h] . K[s]); one
 * d_i-wide key per compressed block, shared by all h_i heads.  No scale.
 * Causal form: page 1, archived_plans/NEXT_STEPS.md, Issue 2 — block s is
 * visible to a query at position p iff ratio*s + ratio - 1 <= p, otherwise
 * its score is -inf.
 *
 * q:      [B][t][h_i][d_i] of dtype, stride_b = q_stride_b elements.
 * w:      [B][t][h_i] float32, stride_b = w_stride_b.
 * k:      [B][n][d_i] of dtype, stride_b = k_stride_b (0 = shared keys).
 * scores: [B][t][ld_s] float32, stride_b = s_stride_b; columns 0..n-1 written.
 * q_pos:  [B][t] int32 device positions for the causal mask, or NULL.
 * Supported: bfloat16 with h_i = 64, d_i = 128 (matrix-core path) and
 *   float32 with h_i <= 64, d_i <= 256, h_i * d_i <= 8192.  n >= 0; ld_s >= n.
 * With bfloat16 and t >= 16 query rows the multi-query scan of section 7
 * runs; every bfloat16 path gives the same bits for the same (query, key).
 * ------------------------------------------------------------------------ */
int csa_index_score(const void *q, const float *w, const void *k, float *scores,
                    csa_dtype dtype, int batch, int t, int h_i, int d_i, int n,
                    const int *q_pos, int ratio, long long q_stride_b, long long w_stride_b,
                    long long k_stride_b, long long s_stride_b, long long ld_s,
                    csa_stream stream);

/* ------------------------------------------------------------------------
 * 2b. FP8 E4M3 indexer keys: quantisation and the FP8 index score.
 *
 * Source: page 1, single_shot_inference.py, comment "B2: FP8 tensor-core
 * scoring path" (indexer keys stored as FP8_E4M3 in the KV cache).  The pages
 * do not spell out the scaling; here every row (a key, or one head of a
 * query) carries one float32 scale and its value is e4m3(code) * scale.
 * E4M3 is the OCP encoding: sign, 4 exponent bits (bias 7), 3 mantissa bits,
 * subnormals, NaN = S.1111.111, no infinity, largest finite 448.
 *
 * csa_quantize_fp8: x [rows][d] float32 or bfloat16 (x_dtype), contiguous ->
 *   codes [rows][d] uint8 and scales [rows] float32: scale = max|row| / 448
 *   (1 for an all-zero row), code = E4M3 of x / scale (binary32 division),
 *   rounded to nearest, ties to the even code, saturating at +-448; -0 keeps
 *   its sign.  NaN inputs are out of contract.  Limits: 1 <= d <= 65536.
 *
 * csa_quantize_query_fp8: a query for the E4M3 score.  q [rows][h][d]
 *   float32 or bfloat16 (q_dtype), contiguous; w [rows][h] float32 head
 *   weights -> q_codes [rows][h][d] uint8 (every head row quantised as
 *   csa_quantize_fp8 quantises a row) and w_folded [rows][h] = w * that head
 *   row's scale (one binary32 multiply; since ReLU(c x) = c ReLU(x) for
 *   c > 0 this carries the query's scale into the score).  Limits as
 *   csa_quantize_fp8, h >= 1.
 *
 * csa_index_score_fp8:
 *   I[t,s] = sum_h w[t,h] * ReLU(k_scale[s] * (e4m3(q[t,h]) . e4m3(k[s])))
 *   q:       [B][t][h_i][d_i] uint8 codes, stride_b = q_stride_b bytes.
 *   w:       [B][t][h_i] float32, stride_b = w_stride_b; a per-head query
 *            scale is folded in by the caller (ReLU(c x) = c ReLU(x), c > 0).
 *   k:       [B][n][d_i] uint8 codes, stride_b = k_stride_b bytes (0 = shared).
 *   k_scale: [B][n] float32, stride_b = ks_stride_b (0 = shared).
 *   scores:  [B][t][ld_s] float32, stride_b = s_stride_b; columns 0..n-1.
 *   q_pos, ratio: the causal form, as for csa_index_score.
 * Supported: h_i = 64, d_i = 128; q, k, w 16-byte aligned and strides that
 * keep them so.  Products of E4M3 values are exact in float32; sums are
 * float32.  From t = 16 query rows per sequence the multi-query form of
 * section 7 runs (same values up to float32 summation order; the key scale
 * is then applied after the head sum, which is exact in real arithmetic
 * since k_scale > 0).
 * ------------------------------------------------------------------------ */
int csa_quantize_fp8(const void *x, csa_dtype x_dtype, unsigned char *codes, float *scales,
                     long long rows, int d, csa_stream stream);
int csa_quantize_query_fp8(const void *q, csa_dtype q_dtype, const float *w, unsigned char *q_codes,
                           float *w_folded, long long rows, int h, int d, csa_stream stream);
int csa_index_score_fp8(const unsigned char *q, const float *w, const unsigned char *k,
                        const float *k_scale, float *scores, int batch, int t, int h_i, int d_i,
                        int n, const int *q_pos, int ratio, long long q_stride_b,
                        long long w_stride_b, long long k_stride_b, long long ks_stride_b,
                        long long s_stride_b, long long ld_s, csa_stream stream);

/* ------------------------------------------------------------------------
 * 2d. FP4 E2M1 indexer keys with E8M0 block scales.
 *
 * Source: page 1, ARCHITECTURE_AND_MEMORY_AUDIT.md, C4 "Optional: Quantize
 * indexer KV to FP4" (an FP4 indexer cache, paired with an FP4 tensor-core
 * scoring kernel, never one without the other).  The pages fix no block
 * layout; here the keys use the formats gfx950's scaled matrix instructions
 * read: E2M1 elements (sign, 2 exponent bits with bias 1, 1 mantissa bit:
 * magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) and one E8M0 scale (2^(s - 127))
 * per 32 consecutive elements; the query stays E4M3 (section 2b).
 *
 * csa_quantize_fp4: x [rows][d] float32 or bfloat16 (x_dtype), contiguous ->
 *   codes [rows][d / 2] bytes (element 2j in the low nibble of byte j,
 *   element 2j + 1 in the high nibble) and scales [rows][d / 32] E8M0 bytes.
 *   A block's scale is 2^X with X the smallest integer such that the
 *   block's largest magnitude is at most 6 * 2^X (so nothing saturates),
 *   clamped to [-127, 127], X = 0 for an all-zero block; each element is
 *   multiplied by 2^-X (exact) and rounded to the nearest E2M1 magnitude,
 *   ties to the even code, its sign kept unless it rounds to zero (code 0).
 *   NaN inputs are out of contract.  Limits: d a multiple of 32, 32 <= d
 *   <= 65536.
 *
 * csa_index_score_fp4:
 *   I[t,s] = sum_h w[t,h] * ReLU(e4m3(q[t,h]) . K[s]),
 *   K[s][j] = e2m1(code[s][j]) * 2^(scale[s][j / 32] - 127).
 *   q:        [B][t][h_i][d_i] uint8 E4M3 codes, stride_b = q_stride_b bytes
 *             (csa_quantize_query_fp8 makes them and the folded weights).
 *   w:        [B][t][h_i] float32, stride_b = w_stride_b, query scales folded in.
 *   k:        [B][n][d_i / 2] packed codes, stride_b = k_stride_b bytes.
 *   k_scales: [B][n] 32-bit words, byte j of word s the scale of elements
 *             32 j .. 32 j + 31 of key s (d_i / 32 = 4 bytes), stride_b =
 *             ks_stride_b words.
 *   scores:   [B][t][ld_s] float32, stride_b = s_stride_b; columns 0..n-1.
 *   q_pos, ratio: the causal form, as for csa_index_score.
 * Supported: h_i = 64, d_i = 128; q, k, w 16-byte aligned and strides that
 * keep them so.  Products of E4M3 and E2M1 values are exact; the matrix
 * core sums in float32 (so the scores agree with the exact sum to float32
 * rounding of partial sums).
 * ------------------------------------------------------------------------ */
int csa_quantize_fp4(const void *x, csa_dtype x_dtype, unsigned char *codes, unsigned char *scales,
                     long long rows, int d, csa_stream stream);
int csa_index_score_fp4(const unsigned char *q, const float *w, const unsigned char *k,
                        const unsigned int *k_scales, float *scores, int batch, int t, int h_i,
                        int d_i, int n, const int *q_pos, int ratio, long long q_stride_b,
                        long long w_stride_b, long long k_stride_b, long long ks_stride_b,
                        long long s_stride_b, long long ld_s, csa_stream stream);

/* ------------------------------------------------------------------------
 * 3. Top-k.
 *
 * Source: page 1, ARCHITECTURE_AND_MEMORY_AUDIT.md, F3 code
 * (tk = min(top_k, n_comp); total.topk(tk, -1)) and page 3,
 * GETTING+CUDAGRAPH_READY.md, Section C item 3 (always k slots, invalid ones
 * masked, no host read of the count).
 *
 * For each of the rows = batch * t score rows (row r of batch b at
 * scores + b * s_stride_b + (r % t) * ld_s), select the k largest valid
 * scores (valid = greater than -inf; NaN is out of contract), ordered by
 * score descending, then index ascending (+0 and -0 are equal).
 * idx:   [B][t][k] int32, unused slots -1.   count: [B][t] int32 = min(k, valid)
 *        (count may be NULL).
 * ws:    csa_topk_workspace_size(batch, t, n, k) bytes of device memory,
 *        16-byte aligned; contents need no initialisation.
 * Limits: 1 <= k <= 2048, 0 <= n < 2^31.
 * ------------------------------------------------------------------------ */
size_t csa_topk_workspace_size(int batch, int t, int n, int k);
int csa_topk(const float *scores, int batch, int t, int n, long long ld_s, long long s_stride_b,
             int k, int *idx, int *count, void *ws, size_t ws_bytes, csa_stream stream);

/* ------------------------------------------------------------------------
 * 4. Gather into gather_buf.
 *
 * Source: page 1 commit message C2 (one preallocated (top_k + window, hd)
 * buffer, filled by slice assignment, no concatenation) and C3 (the SWA ring
 * may wrap); page 1, PERFORMANCE_AUDIT.md, P2 (slot (swa_head + i) % W,
 * swa_len = min(swa_len + T, W)); compressed rows first, then the window
 * (ARCHITECTURE_AND_MEMORY_AUDIT.md, B2).
 *
 * For batch b: rows 0..count[b]-1 of gather_buf are comp_kv[idx[b][j]]
 * (indices clamped to 0..n_comp-1), followed by the swa_len live window rows
 * oldest first: swa[(swa_head - swa_len + j) mod w].  n_valid[b] =
 * count[b] + swa_len.  Rows at and beyond n_valid are not written.
 * comp_kv:    [B][n_comp][d] of dtype, stride kv_stride_b.
 * idx, count: [B][k] and [B] int32 (from csa_topk; count NULL = k).
 * swa:        [B][w][d] of dtype, stride swa_stride_b; swa_head is the next
 *             write slot (0 <= swa_head < w), 0 <= swa_len <= w.
 * gather_buf: [B][k + w][d] of dtype, stride buf_stride_b.
 * n_valid:    [B] int32 (may be NULL).
 * Limits: d * sizeof(dtype) must be a multiple of 16 bytes.
 * ------------------------------------------------------------------------ */
int csa_gather(const void *comp_kv, int n_comp, const int *idx, const int *count, int k,
               const void *swa, int swa_head, int swa_len, int w, void *gather_buf, int *n_valid,
               csa_dtype dtype, int batch, int d, long long kv_stride_b, long long swa_stride_b,
               long long buf_stride_b, csa_stream stream);

/* ------------------------------------------------------------------------
 * 5. Shared-KV sparse attention with a per-head sink.
 *
 * Source: page 1, dsv4/kernels/attention/fmha_6warp_tma_multirow_multitile.cuh,
 * hunk "Sink bias correction (D5c: single softmax over [S_comp, S_swa +
 * sink])": after all rows, M = max(m, sink); the running sum and output are
 * rescaled by exp(m - M) and the sum gains exp(sink - M); the sink has no
 * value row and is already in the scaled domain.  K = V (page 1,
 * PERFORMANCE_AUDIT.md P4; fmha_multitile_op.py, MQA head stride 0).
 *
 * For head h of batch b over rows j < n_valid[b] (clamped to n_max):
 *   s_j = scale * q[h] . kv[j];  M = max(max_j s_j, sink[h]);
 *   out[h] = sum_j exp(s_j - M) kv[j] / (sum_j exp(s_j - M) + exp(sink[h] - M));
 *   lse[h] = M + ln(denominator).  No rows and no sink: out = 0, lse = -inf.
 * q:   [B][h][d] of dtype, stride q_stride_b.     kv: [B][n_max][d] of dtype.
 * sink:[h] float32 or NULL.   out: [B][h][d] of out_dtype.   lse: [B][h] or NULL.
 * ws:  csa_sparse_attn_workspace_size(batch, h, d, n_max) bytes.
 * Supported: bfloat16 with h % 16 == 0, d % 32 == 0, d <= 512;
 *            float32 with d <= 1024, n_max <= 8192.
 * ------------------------------------------------------------------------ */
size_t csa_sparse_attn_workspace_size(int batch, int h, int d, int n_max);
int csa_sparse_attn(const void *q, const void *kv, const int *n_valid, const float *sink,
                    float scale, void *out, float *lse, csa_dtype dtype, csa_dtype out_dtype,
                    int batch, int h, int d, int n_max, long long q_stride_b,
                    long long kv_stride_b, long long out_stride_b, void *ws, size_t ws_bytes,
                    csa_stream stream);

/* ------------------------------------------------------------------------
 * 6. One decode step of one CSA layer.
 *
 * Source: page 2 (compare master..pure-nvfp4), single_shot_inference.py,
 * eager_attention: append the new token's KV to the SWA ring, run the main
 * compressor and the indexer's key compressor, indexer top-k, gather, then
 * attention.  The compressors emit an entry only when the token completes a
 * block (page 1, PERFORMANCE_AUDIT.md P7): pos % m == m - 1.
 *
 * The layer state is host-known integers plus caller-owned device caches.
 * The call enqueues, in stream order:
 *   a. swa[swa_head] = kv_new (every batch element);
 *   b. if pos % m == m - 1: comp_kv[n_comp] = compress(z_main, c_main) and
 *      idx_keys[n_comp] = compress(z_idx, c_idx) (overlap convention as in
 *      csa_compress, with first_block = pos / m);
 *   c. scores over the N = n_comp (+1 if b ran) keys, top-k, gather, attention.
 * With mixed main KV (kv_dtype = CSA_FP8_E4M3, section 6c) step a packs
 * kv_new (already rotated) into its ring record, step b packs the
 * compressed entry with its RoPE dims rotated by comp_rope row pos / m, the
 * attention decodes the records (E4M3 times scale, rounded to bfloat16) and
 * the output's RoPE dims are rotated back by rope row pos; gather_buf holds
 * records (gather_stride_b in bytes).
 * With E4M3 indexer keys (idx_dtype = CSA_FP8_E4M3; bfloat16 caches, h_i = 64,
 * d_i = 128) step b stores the compressed key as csa_quantize_fp8 would
 * (codes into idx_keys[n_comp], its scale into idx_scales[n_comp]); step c
 * takes the bfloat16 q_idx and plain w_idx, quantises every head row of
 * q_idx and folds its scale into that head's weight exactly as
 * csa_quantize_query_fp8 does, and scores as csa_index_score_fp8 does.
 * Section 2c (idx_rescore = k_cand > 0, E4M3 keys only): step b also stores
 * the new key in bfloat16 in idx_keys_exact[n_comp] (the bfloat16 step's
 * rounding); step c writes the E4M3 scores to io->scores, takes the k_cand
 * best of them (the top-k rules), computes their exact scores from
 * idx_keys_exact and the bfloat16 query (the same values the bfloat16 step
 * computes for those keys) and selects the top_k best of those (score
 * descending, lower index first).  Source of the two stages: the recall
 * gate of page 1, ARCHITECTURE_AND_MEMORY_AUDIT.md (Tier 1 gate 4: the
 * selection must keep 99% of the exact top-512), which per-row E4M3 alone
 * misses on crowded scores (93.6% on the 1M-context workload).  Host
 * counters only (csa_decode_step_dev: CSA_ERR_UNSUPPORTED).
 * With E2M1 indexer keys (idx_dtype = CSA_FP4_E2M1, section 2d; same
 * conditions as E4M3 keys) step b stores the compressed key as
 * csa_quantize_fp4 would (packed codes into idx_keys[n_comp], its four
 * E8M0 scales into the 32-bit word idx_scales[n_comp]) and step c scores as
 * csa_index_score_fp4 does, with the query quantised as for E4M3 keys;
 * idx_rescore works as for E4M3 keys (E2M1 keys alone keep about 80% of the
 * exact top-512 on the 1M-context workload; the 2048 best by E2M1 score,
 * rescored, keep all of it).
 * It does NOT update the host integers: afterwards the caller sets
 * swa_head = (swa_head + 1) % w, swa_len = min(swa_len + 1, w) and, if a block
 * completed, n_comp += 1 (csa_layer_advance does exactly this).
 * ------------------------------------------------------------------------ */
typedef struct csa_layer_desc {
    int batch;       /* sequences, each with its own caches             */
    int h, d;        /* main attention heads and head dim (K = V)       */
    int h_i, d_i;    /* indexer heads and key width                     */
    int m;           /* compression ratio                               */
    int w;           /* SWA window                                      */
    int top_k;
    int overlap;     /* 0: plain ratio-m blocks; 1: overlapped a|b form */
    csa_dtype dtype; /* storage of q, q_idx, kv_new and all caches      */
    csa_dtype out_dtype;
    void *comp_kv;  long long comp_kv_stride_b;   /* [B][max_comp][d]   */
    void *idx_keys; long long idx_keys_stride_b;  /* [B][max_comp][d_i] */
    void *swa;      long long swa_stride_b;       /* [B][w][d]          */
    int max_comp;
    const float *main_bias; /* [m][d] (overlap: [m][2d])     */
    const float *idx_bias;  /* [m][d_i] (overlap: [m][2d_i]) */
    const float *main_norm; /* [d] or NULL   */
    const float *idx_norm;  /* [d_i] or NULL */
    const float *sink;      /* [h] or NULL   */
    float scale;            /* attention logit scale (usually 1/sqrt(d)) */
    int n_comp;             /* compressed entries before this step */
    int swa_head;           /* next SWA write slot */
    int swa_len;            /* live SWA rows */
    /* E4M3 indexer keys (section 2b; appended, so a zero-filled descriptor
     * keeps keys of `dtype`): idx_dtype = CSA_FP8_E4M3 makes idx_keys
     * [B][max_comp][d_i] uint8 codes (idx_keys_stride_b in bytes) with row
     * scales idx_scales [B][max_comp] float32 (stride idx_scales_stride_b);
     * q_idx stays bfloat16 [B][h_i][d_i] (the step quantises it).  Any other
     * value: keys stored as `dtype`. */
    csa_dtype idx_dtype;
    float *idx_scales; long long idx_scales_stride_b;
    /* (idx_dtype = CSA_FP4_E2M1, section 2d: idx_keys [B][max_comp][d_i / 2]
     * packed E2M1 codes (stride in bytes); idx_scales [B][max_comp] 32-bit
     * words of four E8M0 block scales (stride in words); d_i = 128) */
    /* Mixed main KV (section 6c; appended: zero keeps comp_kv / swa rows of
     * `dtype`): kv_dtype = CSA_FP8_E4M3 makes every comp_kv and swa row a
     * 592-byte record (csa_pack_kv_mixed), comp_kv_stride_b and swa_stride_b
     * in bytes.  rope_cos / rope_sin: [rope_rows][rope_dim / 2] float32, the
     * table rows of token positions; comp_rope_cos / comp_rope_sin:
     * [comp_rope_rows][rope_dim / 2], the rows of compressed entries by block
     * index (pos / m). */
    csa_dtype kv_dtype;
    int rope_dim;
    const float *rope_cos, *rope_sin; int rope_rows;
    const float *comp_rope_cos, *comp_rope_sin; int comp_rope_rows;
    /* Recall-restored E4M3 or E2M1 keys (section 2c; appended: zero = off): with
     * idx_dtype = CSA_FP8_E4M3 or CSA_FP4_E2M1 and idx_rescore = k_cand (top_k <= k_cand <=
     * 2048) the layer also keeps its keys as bfloat16 in idx_keys_exact
     * [B][max_comp][d_i] (stride idx_keys_exact_stride_b elements, 16-byte
     * aligned rows). */
    int idx_rescore;
    void *idx_keys_exact; long long idx_keys_exact_stride_b;
} csa_layer_desc;

typedef struct csa_step_io {
    int pos;                                          /* position of the new token   */
    const void *q;      long long q_stride_b;         /* [B][h][d]                   */
    const void *q_idx;  long long q_idx_stride_b;     /* [B][h_i][d_i]               */
    const float *w_idx; long long w_stride_b;         /* [B][h_i]                    */
    const void *kv_new; long long kv_new_stride_b;    /* [B][d]                      */
    /* rows of the block this token completes (read only when it does):
     * overlap 0: [B][m][d] / [B][m][d_i]; overlap 1: [B][2m][2d] / [B][2m][2d_i]
     * holding block pos/m - 1 then block pos/m (block 0: its m rows only).   */
    const float *z_main, *c_main; long long zc_main_stride_b;
    const float *z_idx,  *c_idx;  long long zc_idx_stride_b;
    /* outputs (device, caller-owned) */
    float *scores;      long long scores_stride_b;    /* [B][>= N] float32           */
    int *topk_idx;                                    /* [B][top_k]                  */
    int *topk_count;                                  /* [B]                         */
    void *gather_buf;   long long gather_stride_b;    /* [B][top_k + w][d] of dtype  */
    int *n_valid;                                     /* [B]                         */
    void *out;          long long out_stride_b;       /* [B][h][d] of out_dtype      */
    float *lse;                                       /* [B][h] or NULL              */
} csa_step_io;

size_t csa_decode_step_workspace_size(const csa_layer_desc *layer);
int csa_decode_step(const csa_layer_desc *layer, const csa_step_io *io, void *ws,
                    size_t ws_bytes, csa_stream stream);

/* ------------------------------------------------------------------------
 * 6f. The decode step in two calls.
 *
 * Source: as section 6 (page 2, single_shot_inference.py, eager_attention):
 * the step's first part reads the new token's inputs and the indexer keys,
 * its second part the selected compressed rows and the window.
 *
 * csa_decode_step_scan enqueues steps a and b and the index score of step c
 * (one kernel on the bfloat16 paths: the SWA append, the compression of a
 * completed block, the scan over every key with each workgroup's top-k
 * candidates written to the workspace); csa_decode_step_attend enqueues the
 * rest of step c (top-k, gather, attention).  Called in that order on one
 * stream with the same layer, io and workspace (the candidates pass through
 * it), they do exactly what one csa_decode_step call does, with the same
 * validation and errors.  Independent work may be enqueued between them; the
 * workspace must not be touched in between.
 * ------------------------------------------------------------------------ */
int csa_decode_step_scan(const csa_layer_desc *layer, const csa_step_io *io, void *ws,
                         size_t ws_bytes, csa_stream stream);
int csa_decode_step_attend(const csa_layer_desc *layer, const csa_step_io *io, void *ws,
                           size_t ws_bytes, csa_stream stream);

/* ------------------------------------------------------------------------
 * 6e. The decode step with no workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).
 *
 * csa_decode_step_noalloc runs exactly csa_decode_step (same kernels, same
 * results) with its scratch in a fixed device array inside the library:
 * csa_decode_step_noalloc_max_bytes() bytes (32 MiB), one copy per GPU,
 * held from the first call on that GPU until the process ends.  The caller
 * still owns and passes every input and output (layer caches, io).  It
 * calls no allocating routine.  A layer whose step needs more scratch than
 * that (csa_decode_step_workspace_size(layer) > the maximum, e.g. more
 * than 8 sequences at top_k 512 + window 128, d 512) is rejected with
 * CSA_ERR_WORKSPACE before anything is enqueued.  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from different host threads without stream
 * ordering between them) race on it and give undefined results.  Nothing
 * in the array needs to start at zero.
 * ------------------------------------------------------------------------ */
size_t csa_decode_step_noalloc_max_bytes(void);
int csa_decode_step_noalloc(const csa_layer_desc *layer, const csa_step_io *io, csa_stream stream);

/* ------------------------------------------------------------------------
 * 6d. The decode step with its counters on the device (graph replay).
 *
 * Source: page 3, GETTING+CUDAGRAPH_READY.md, Section C: the compressor runs
 * every step into a persistent partial state and emits its entry on the
 * block boundary device-side (item 1), fixed shapes with masking (items 2,
 * 3), positions advanced on the device (item 5).
 *
 * csa_decode_step_dev runs the same step as csa_decode_step, but reads pos,
 * n_comp, swa_head and swa_len from `state` (device memory) when its kernels
 * run, decides there whether the token completes a block, and advances the
 * state afterwards (pos + 1; n_comp + 1 after a completed block; the SWA
 * ring as csa_layer_advance does).  One captured graph of it therefore
 * replays step after step with nothing decided on the host.  The layer's
 * host counters and io->pos are ignored.  Differences from csa_decode_step:
 *   - io->z_main, c_main, z_idx, c_idx are this token's rows only: [B][d]
 *     and [B][d_i] (overlap 1: [B][2d], [B][2d_i]), every step; the step keeps
 *     the rows of the current and the previous block in `ring`
 *     (csa_decode_step_dev_ring_size bytes of caller-owned device memory, no
 *     initialisation needed beyond what the steps themselves write: the
 *     first block of a layer must be stepped from its first token);
 *   - scores must hold max_comp columns per sequence;
 *   - a completed block that finds the cache full (n_comp == max_comp)
 *     writes nothing and sets bit 0 of state->flags;
 *   - with mixed KV, positions and blocks past the RoPE tables use the
 *     tables' last rows;
 *   - bfloat16 caches only (CSA_ERR_UNSUPPORTED otherwise); E4M3 indexer
 *     keys and mixed main KV as for csa_decode_step.
 * The workspace is csa_decode_step_workspace_size(layer) bytes.
 * ------------------------------------------------------------------------ */
typedef struct csa_dev_state {
    int pos, n_comp, swa_head, swa_len, flags;
} csa_dev_state;
size_t csa_decode_step_dev_ring_size(const csa_layer_desc *layer);
int csa_decode_step_dev(const csa_layer_desc *layer, const csa_step_io *io, csa_dev_state *state,
                        float *ring, size_t ring_bytes, void *ws, size_t ws_bytes, csa_stream stream);

/* Advance the host-known counters of `layer` past a step at position pos. */
int csa_layer_advance(csa_layer_desc *layer, int pos);

/* ------------------------------------------------------------------------
 * 6c. Mixed main KV: E4M3 NoPE codes + bfloat16 RoPE part per row.
 *
 * Source: page 2, single_shot_inference.py, eager_attention (the "B1
 * storage-native mixed path": kv_quantize's quantize_fp8_e4m3_from_fp32 of
 * the NoPE part, the RoPE part kept in bfloat16 and rotated at the
 * compressed entry's position, the FMHA over the mixed rows, then "Inverse
 * RoPE" of the output); the RoPE pairing of page 1, PERFORMANCE_AUDIT.md P5
 * (even / odd entries of the trailing rope_dim; inverse (e c + o s,
 * -e s + o c), forward its inverse).
 *
 * Record of one row (d = 512, rope_dim = 64), 592 bytes, 16-byte aligned:
 *   bytes 0..447 E4M3 codes of entries 0..447 (as csa_quantize_fp8: scale =
 *   max|x| / 448 over those entries, 1 if all zero, nearest-even codes),
 *   bytes 448..575 entries 448..511 as bfloat16 (nearest even),
 *   bytes 576..579 the float32 scale, bytes 580..591 zero.
 *
 * csa_pack_kv_mixed: x [rows][512] float32 or bfloat16, contiguous ->
 *   rec [rows][592] bytes (no rotation: rows are taken as already rotated).
 * ------------------------------------------------------------------------ */
int csa_pack_kv_mixed(const void *x, csa_dtype x_dtype, unsigned char *rec, long long rows, int d,
                      int rope_dim, csa_stream stream);

/* ------------------------------------------------------------------------
 * 6b. One decode step of an HCA layer (heavily compressed attention).
 *
 * Source: page 1, PERFORMANCE_AUDIT.md, the forward_attention branches —
 * layers with a compression ratio above 4 attend to ALL compressed entries
 * followed by the SWA window (torch.cat([kv_cache.comp_kv, swa_kv])); page 2,
 * single_shot_inference.py, eager_attention (gather_mixed_all for ratio > 4);
 * the non-overlapped compressor of page 1, hca_compress_reduce_kernel.
 *
 * The same descriptor and io as csa_decode_step, with the indexer fields
 * ignored (idx_keys, idx_bias, idx_norm, h_i, d_i, top_k; q_idx, w_idx,
 * z_idx, c_idx, scores, topk_idx, topk_count, gather_buf).  Enqueues:
 *   a. swa[swa_head] = kv_new;
 *   b. if pos % m == m - 1: comp_kv[n_comp] = compress(z_main, c_main)
 *      (overlap must be 0);
 *   c. one softmax (scale, sink in the denominator) over comp_kv[0 .. N)
 *      then the live window, N = n_comp (+1 if b ran); out [B][h][d],
 *      lse [B][h] (nullable), n_valid [B] = N + window rows (nullable).
 * bfloat16 caches only (CSA_ERR_UNSUPPORTED otherwise); h a multiple of 16,
 * d a multiple of 32 up to 512, max_comp + w <= 8192.  The host integers are
 * advanced by the caller (csa_layer_advance) as for csa_decode_step.
 * Mixed main KV (kv_dtype = CSA_FP8_E4M3, section 6c): the records, tables
 * and checks of csa_decode_step's mixed form, without a main norm
 * (main_norm must be null: CSA_ERR_UNSUPPORTED); the ring record and the
 * entry's record (rotated at block pos / m) are packed as there, every row
 * is decoded to bfloat16 for the softmax, and out's RoPE dims are rotated
 * back at pos.
 * Workspace: csa_hca_decode_step_workspace_size(layer) bytes, 16-byte aligned.
 * ------------------------------------------------------------------------ */
size_t csa_hca_decode_step_workspace_size(const csa_layer_desc *layer);
int csa_hca_decode_step(const csa_layer_desc *layer, const csa_step_io *io, void *ws,
                        size_t ws_bytes, csa_stream stream);

/* ------------------------------------------------------------------------
 * 6g. The HCA step with its counters on the device (graph replay).
 *
 * Source: page 3, GETTING+CUDAGRAPH_READY.md, Section C item 1 (the
 * compressors' periodic host branch, 3/4 for CSA and 127/128 for HCA,
 * becomes a persistent partial state with a device-side emit on the block
 * boundary), items 2, 3 and 5, as for csa_decode_step_dev.
 *
 * csa_hca_decode_step_dev runs the same step as csa_hca_decode_step, with
 * pos, n_comp, swa_head and swa_len read from `state` when its kernels run,
 * the block boundary (pos % m == m - 1, with room in the cache) decided
 * there, and the state advanced afterwards as csa_decode_step_dev advances
 * it.  io->z_main, c_main are this token's rows only ([B][d]), every step;
 * the step keeps the rows of the current and the previous block in `ring`
 * (csa_hca_decode_step_dev_ring_size bytes of caller-owned device memory;
 * the first block of a layer must be stepped from its first token).  A
 * completed block that finds the cache full writes nothing and sets bit 0
 * of state->flags.  With mixed KV, positions and blocks past the RoPE tables
 * use the tables' last rows.  Other arguments, limits and errors as
 * csa_hca_decode_step; the workspace is csa_hca_decode_step_workspace_size.
 * ------------------------------------------------------------------------ */
size_t csa_hca_decode_step_dev_ring_size(const csa_layer_desc *layer);
int csa_hca_decode_step_dev(const csa_layer_desc *layer, const csa_step_io *io, csa_dev_state *state,
                            float *ring, size_t ring_bytes, void *ws, size_t ws_bytes, csa_stream stream);

/* ------------------------------------------------------------------------
 * 7. Prefill-shaped chunk: t query tokens at positions pos0, pos0+1, ...
 *    against one compressed history.
 *
 * Sources: the index score and its causal mask as in section 2; the
 * fixed-shape top-k of section 3; the per-query composition of page 2,
 * single_shot_inference.py, eager_attention (score -> top-k -> one softmax
 * over the selected compressed rows, then the sliding window, plus the sink
 * of the D5c hunk on page 1).  The history holds the chunk's own blocks too:
 * the causal mask hides each block until the query that completes it.  The
 * window of the query at position p is the raw KV of positions
 * max(0, p - window + 1) .. p, oldest first (the decode step's SWA window,
 * applied per query).
 *
 * csa_index_topk: score + causal mask + top-k for every query, bfloat16 keys
 *   and queries (h_i = 64, d_i = 128), without holding all t x n scores:
 *   at most 256 query rows of scores live in the workspace at a time.
 *   q: [t][64][128] bf16, w: [t][64] float32, k: [n][128] bf16 (16-byte
 *   aligned); pos0 >= 0 gives query row r the position pos0 + r (pos0 < 0:
 *   no mask).  idx: [t][top_k] int32 out (rank order: score descending,
 *   lower index first on ties; -1 past the count), count: [t] int32 out
 *   (nullable) = min(top_k, visible blocks).  1 <= top_k <= 2048.
 *   ws: csa_index_topk_workspace_size(t, n, top_k) bytes, 16-byte aligned.
 *
 * csa_index_topk_fp8: the same over E4M3 queries and keys (section 2b):
 *   q: [t][64][128] uint8 codes, w: [t][64] float32 with the query's per-head
 *   scales folded in, k: [n][128] uint8 codes, k_scale: [n] float32 row
 *   scales; scores as csa_index_score_fp8 computes them.  The same workspace
 *   size, outputs and limits as csa_index_topk.
 *
 * csa_index_topk_fp8_rescored: the two-stage E4M3 selection of section 2c
 *   for every query: q [t][64][128] bf16 and w [t][64] float32 (plain
 *   weights; the query is quantised as csa_quantize_query_fp8 does), k8 /
 *   k_scale [n][128] codes and [n] scales, k16 [n][128] the same keys in
 *   bfloat16.  Per query, the k_cand best by E4M3 score (csa_index_topk_fp8),
 *   then their exact scores from k16 and the bfloat16 query (the values
 *   csa_index_score computes) and the top_k best of those: idx [t][top_k]
 *   (score descending, lower index first, -1 past the count), count [t]
 *   (nullable) = min(top_k, visible blocks).  top_k <= k_cand <= 2048.
 *   ws: csa_index_topk_fp8_rescored_workspace_size(t, n, top_k, k_cand)
 *   bytes, 16-byte aligned.
 *
 * csa_index_topk_fp4 / csa_index_topk_fp4_rescored: the same two calls over
 *   FP4 keys (section 2d; page 1, ARCHITECTURE_AND_MEMORY_AUDIT.md, C4):
 *   k / k4 [n][64] packed E2M1 codes and k_scales [n] 32-bit words of four
 *   E8M0 block scales, as csa_quantize_fp4 writes them (its [n][4] bytes);
 *   scores as csa_index_score_fp4 computes them.  Query, outputs, limits
 *   and workspace sizes as their E4M3 forms (the rescored one sizes its
 *   workspace with csa_index_topk_fp8_rescored_workspace_size).  FP4 keys
 *   alone keep about 80% of the exact top-512 at 250,000 keys; the
 *   two-stage form restores it with k_cand = 4 top_k.
 *
 * csa_prefill_attn: per query row r, one softmax (scale, then the sink in the
 *   denominator only) over comp_kv[idx[r][0 .. count[r])] followed by its
 *   window rows.  q: [t][h][d] bf16; comp_kv: [n_comp][d] bf16; idx/count as
 *   csa_index_topk writes them (count nullable: k rows; indices outside
 *   0..n_comp-1 are clamped); win_kv: [t + window - 1][d] bf16, row i
 *   holding position pos0 - window + 1 + i (rows of negative positions are
 *   never read); sink: [h] float32 or NULL; out: [t][h][d] of out_dtype
 *   (float32 or bfloat16); lse: [t][h] float32 (sink included) or NULL.
 *   Supported: h a multiple of 16 up to 64, d in {128, 256, 512},
 *   pos0 >= 0, window >= 1, 1 <= k <= 2048.  No workspace.
 *
 * Both only enqueue work on `stream`; all pointers are device memory owned
 * by the caller.  Errors: CSA_ERR_INVALID_ARG for null/misaligned pointers
 * or out-of-range sizes, CSA_ERR_UNSUPPORTED for other head/width shapes,
 * CSA_ERR_WORKSPACE for a short workspace, CSA_ERR_LAUNCH on launch failure.
 * ------------------------------------------------------------------------ */
size_t csa_index_topk_workspace_size(int t, int n, int top_k);
int csa_index_topk(const void *q, const float *w, const void *k, int t, int h_i, int d_i, int n,
                   long long pos0, int ratio, int top_k, int *idx, int *count, void *ws,
                   size_t ws_bytes, csa_stream stream);
int csa_index_topk_fp8(const unsigned char *q, const float *w, const unsigned char *k,
                       const float *k_scale, int t, int h_i, int d_i, int n, long long pos0,
                       int ratio, int top_k, int *idx, int *count, void *ws, size_t ws_bytes,
                       csa_stream stream);
size_t csa_index_topk_fp8_rescored_workspace_size(int t, int n, int top_k, int k_cand);
int csa_index_topk_fp8_rescored(const void *q, const float *w, const unsigned char *k8, const float *k_scale,
                                const void *k16, int t, int h_i, int d_i, int n, long long pos0, int ratio,
                                int top_k, int k_cand, int *idx, int *count, void *ws, size_t ws_bytes,
                                csa_stream stream);
int csa_index_topk_fp4(const unsigned char *q, const float *w, const unsigned char *k,
                       const unsigned int *k_scales, int t, int h_i, int d_i, int n, long long pos0,
                       int ratio, int top_k, int *idx, int *count, void *ws, size_t ws_bytes,
                       csa_stream stream);
int csa_index_topk_fp4_rescored(const void *q, const float *w, const unsigned char *k4,
                                const unsigned int *k_scales, const void *k16, int t, int h_i, int d_i,
                                int n, long long pos0, int ratio, int top_k, int k_cand, int *idx,
                                int *count, void *ws, size_t ws_bytes, csa_stream stream);
int csa_prefill_attn(const void *q, const void *comp_kv, int n_comp, const int *idx,
                     const int *count, int k, const void *win_kv, int window, long long pos0,
                     const float *sink, float scale, void *out, csa_dtype out_dtype, float *lse,
                     int t, int h, int d, csa_stream stream);

/* csa_prefill_attn_mixed: csa_prefill_attn over mixed main KV (section 6c;
 *   page 2, single_shot_inference.py, eager_attention, the storage-native
 *   mixed gather, and its inverse RoPE on the output).  d = 512.
 *   comp_rec: [n_comp][592] records; win_rec: [t + window - 1][592] records,
 *   row i holding position pos0 - window + 1 + i; every row attended is the
 *   record's decoded value (E4M3 code times the row scale, bf16 RoPE part).
 *   rope_cos / rope_sin: float32 [rope_rows][32]; out's RoPE dims (the last
 *   64, (even, odd) pairs) are rotated back by row pos0 + r for query row r,
 *   so pos0 + t <= rope_rows.  Other arguments, limits and errors as
 *   csa_prefill_attn (h a multiple of 16 up to 64); null tables or
 *   misaligned records: CSA_ERR_INVALID_ARG.  No workspace. */
int csa_prefill_attn_mixed(const void *q, const unsigned char *comp_rec, int n_comp, const int *idx,
                           const int *count, int k, const unsigned char *win_rec, int window,
                           long long pos0, const float *rope_cos, const float *rope_sin, int rope_rows,
                           const float *sink, float scale, void *out, csa_dtype out_dtype, float *lse,
                           int t, int h, csa_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H */

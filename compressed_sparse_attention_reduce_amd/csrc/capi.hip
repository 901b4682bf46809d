// C ABI of the CSA decode path (declared in include/csa.h).
//
// This layer validates host-known arguments, sizes workspaces and enqueues
// the kernels of compress.hip, index_score.hip, topk.hip, gather.hip and
// attn.hip on the caller's stream.  It never synchronises, never reads device
// memory and never allocates.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <mutex>

#include "../../include/csa.h"
#include "kernels.h"
#include "prefill.h"

namespace csa {

int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    if (dev >= 0 && dev < 64) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

}  // namespace csa

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return CSA_OK;
}

int launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(CSA_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

#define CHECK(cond, ...)                                            \
    do {                                                            \
        if (!(cond)) return fail(CSA_ERR_INVALID_ARG, __VA_ARGS__); \
    } while (0)

int elem_size(csa_dtype dt) { return dt == CSA_BF16 ? 2 : 4; }
bool dtype_ok(int dt) { return dt == CSA_F32 || dt == CSA_BF16; }

}  // namespace

extern "C" {

const char* csa_last_error(void) { return g_err; }

int csa_compress(const float* z, const float* c, const float* bias, const float* norm_w, void* out,
                 csa_dtype out_dtype, int batch, int n_blocks, int m, int d, int overlap,
                 int first_block, long long zc_stride_b, long long out_stride_b, csa_stream stream) {
    CHECK(z && c && bias && out, "csa_compress: null pointer argument");
    CHECK(dtype_ok(out_dtype), "csa_compress: bad out_dtype %d", (int)out_dtype);
    CHECK(batch >= 1 && n_blocks >= 0, "csa_compress: batch %d / n_blocks %d", batch, n_blocks);
    CHECK(m >= 1 && m <= 1024, "csa_compress: m=%d out of 1..1024", m);
    CHECK(d >= 1 && d <= 4096, "csa_compress: d=%d out of 1..4096", d);
    CHECK(overlap == 0 || overlap == 1, "csa_compress: overlap must be 0 or 1");
    CHECK(first_block >= 0, "csa_compress: first_block < 0");
    CHECK(zc_stride_b >= 0 && out_stride_b >= 0, "csa_compress: negative stride");
    CHECK(batch == 1 || (zc_stride_b > 0 && out_stride_b > 0), "csa_compress: zero batch stride");
    return launched(csa::launch_compress(z, c, bias, norm_w, out, out_dtype == CSA_BF16, batch,
                                         n_blocks, m, d, overlap != 0, first_block, zc_stride_b,
                                         out_stride_b, static_cast<hipStream_t>(stream)),
                    "csa_compress");
}

static int check_score_args(const void* q, const float* w, const void* k, float* scores,
                            csa_dtype dtype, int batch, int t, int h_i, int d_i, int n, int ratio,
                            long long q_stride_b, long long w_stride_b, long long k_stride_b,
                            long long s_stride_b, long long ld_s, const char* who) {
    CHECK(q && w && k && scores, "%s: null pointer argument", who);
    CHECK(dtype_ok(dtype), "%s: bad dtype %d", who, (int)dtype);
    CHECK(batch >= 1 && t >= 1 && n >= 0, "%s: batch %d t %d n %d", who, batch, t, n);
    CHECK(batch * static_cast<long long>(t) <= 65535, "%s: batch*t above 65535", who);
    CHECK(ratio >= 1, "%s: ratio %d", who, ratio);
    CHECK(ld_s >= n && q_stride_b >= 0 && w_stride_b >= 0 && k_stride_b >= 0 && s_stride_b >= 0,
          "%s: bad strides", who);
    if (dtype == CSA_BF16) {
        if (h_i != 64 || d_i != 128)
            return fail(CSA_ERR_UNSUPPORTED, "%s: bf16 path needs h_i=64, d_i=128 (got %d, %d)", who, h_i, d_i);
        CHECK(aligned16(q) && aligned16(k) && aligned16(w), "%s: q, k, w must be 16-byte aligned", who);
        CHECK(q_stride_b % 8 == 0 && k_stride_b % 8 == 0 && w_stride_b % 4 == 0,
              "%s: batch strides must keep 16-byte alignment", who);
    } else {
        if (h_i < 1 || h_i > 64 || d_i < 1 || d_i > 256 || h_i * d_i > 8192)
            return fail(CSA_ERR_UNSUPPORTED, "%s: f32 path needs 1<=h_i<=64, 1<=d_i<=256, h_i*d_i<=8192", who);
    }
    return CSA_OK;
}

int csa_index_score(const void* q, const float* w, const void* k, float* scores, csa_dtype dtype,
                    int batch, int t, int h_i, int d_i, int n, const int* q_pos, int ratio,
                    long long q_stride_b, long long w_stride_b, long long k_stride_b,
                    long long s_stride_b, long long ld_s, csa_stream stream) {
    const int rc = check_score_args(q, w, k, scores, dtype, batch, t, h_i, d_i, n, ratio, q_stride_b,
                                    w_stride_b, k_stride_b, s_stride_b, ld_s, "csa_index_score");
    if (rc != CSA_OK) return rc;
    csa::ScoreArgs a{q, w, k, scores, batch, t, h_i, d_i, n, q_pos, ratio,
                     q_stride_b, w_stride_b, k_stride_b, s_stride_b, ld_s, csa::CandArgs{nullptr, 0, 0}};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == CSA_BF16 && t >= csa::kMqMinRows)
        return launched(csa::launch_index_score_mq(a, -1, s), "csa_index_score");
    return launched(dtype == CSA_BF16 ? csa::launch_index_score_bf16(a, nullptr, s)
                                      : csa::launch_index_score_f32(a, s),
                    "csa_index_score");
}

int csa_quantize_fp8(const void* x, csa_dtype x_dtype, unsigned char* codes, float* scales, long long rows,
                     int d, csa_stream stream) {
    CHECK((x && codes && scales) || rows == 0, "csa_quantize_fp8: null pointer argument");
    CHECK(x_dtype == CSA_F32 || x_dtype == CSA_BF16, "csa_quantize_fp8: x must be float32 or bfloat16");
    CHECK(rows >= 0 && rows <= (1LL << 31) * 64, "csa_quantize_fp8: rows %lld", rows);
    CHECK(d >= 1 && d <= 65536, "csa_quantize_fp8: d=%d out of 1..65536", d);
    return launched(csa::launch_quantize_fp8(x, x_dtype == CSA_BF16, codes, scales, rows, d,
                                             static_cast<hipStream_t>(stream)),
                    "csa_quantize_fp8");
}

int csa_quantize_fp4(const void* x, csa_dtype x_dtype, unsigned char* codes, unsigned char* scales, long long rows,
                     int d, csa_stream stream) {
    CHECK((x && codes && scales) || rows == 0, "csa_quantize_fp4: null pointer argument");
    CHECK(x_dtype == CSA_F32 || x_dtype == CSA_BF16, "csa_quantize_fp4: x must be float32 or bfloat16");
    CHECK(rows >= 0 && rows <= (1LL << 31) * 4, "csa_quantize_fp4: rows %lld", rows);
    CHECK(d >= 32 && d <= 65536 && d % 32 == 0, "csa_quantize_fp4: d=%d (a multiple of 32 in 32..65536)", d);
    return launched(csa::launch_quantize_fp4(x, x_dtype == CSA_BF16, codes, scales, rows, d,
                                             static_cast<hipStream_t>(stream)),
                    "csa_quantize_fp4");
}

static int check_fp8_score_args(const void* q, const float* w, const void* k, const float* k_scale, float* scores,
                                int batch, int t, int h_i, int d_i, int n, int ratio, long long q_stride_b,
                                long long w_stride_b, long long k_stride_b, long long ks_stride_b,
                                long long s_stride_b, long long ld_s, const char* who) {
    CHECK(q && w && k && k_scale && scores, "%s: null pointer argument", who);
    CHECK(batch >= 1 && t >= 1 && n >= 0, "%s: batch %d t %d n %d", who, batch, t, n);
    CHECK(batch * static_cast<long long>(t) <= 65535, "%s: batch*t above 65535", who);
    CHECK(ratio >= 1, "%s: ratio %d", who, ratio);
    CHECK(ld_s >= n && q_stride_b >= 0 && w_stride_b >= 0 && k_stride_b >= 0 && ks_stride_b >= 0 &&
              s_stride_b >= 0,
          "%s: bad strides", who);
    if (h_i != 64 || d_i != 128)
        return fail(CSA_ERR_UNSUPPORTED, "%s: E4M3 and E2M1 keys need h_i=64, d_i=128 (got %d, %d)", who, h_i, d_i);
    CHECK(aligned16(q) && aligned16(k) && aligned16(w), "%s: q, k, w must be 16-byte aligned", who);
    CHECK(q_stride_b % 16 == 0 && k_stride_b % 16 == 0 && w_stride_b % 4 == 0,
          "%s: batch strides must keep 16-byte alignment", who);
    return CSA_OK;
}

int csa_quantize_query_fp8(const void* q, csa_dtype q_dtype, const float* w, unsigned char* q_codes, float* w_folded,
                           long long rows, int h, int d, csa_stream stream) {
    CHECK((q && w && q_codes && w_folded) || rows == 0, "csa_quantize_query_fp8: null pointer argument");
    CHECK(q_dtype == CSA_F32 || q_dtype == CSA_BF16, "csa_quantize_query_fp8: q must be float32 or bfloat16");
    CHECK(rows >= 0 && h >= 1 && static_cast<long long>(rows) * h <= (1LL << 31) * 64,
          "csa_quantize_query_fp8: rows %lld h %d", rows, h);
    CHECK(d >= 1 && d <= 65536, "csa_quantize_query_fp8: d=%d out of 1..65536", d);
    return launched(csa::launch_quantize_fp8(q, q_dtype == CSA_BF16, q_codes, nullptr, rows * h, d,
                                             static_cast<hipStream_t>(stream), w, w_folded),
                    "csa_quantize_query_fp8");
}

int csa_pack_kv_mixed(const void* x, csa_dtype x_dtype, unsigned char* rec, long long rows, int d, int rope_dim,
                      csa_stream stream) {
    CHECK((x && rec) || rows == 0, "csa_pack_kv_mixed: null pointer argument");
    CHECK(x_dtype == CSA_F32 || x_dtype == CSA_BF16, "csa_pack_kv_mixed: x must be float32 or bfloat16");
    CHECK(rows >= 0 && rows <= (1LL << 31) * 4, "csa_pack_kv_mixed: rows %lld", rows);
    if (d != csa::kMixD || rope_dim != csa::kMixRope)
        return fail(CSA_ERR_UNSUPPORTED, "csa_pack_kv_mixed: needs d = %d, rope_dim = %d", csa::kMixD,
                    csa::kMixRope);
    CHECK(aligned16(rec) || rows == 0, "csa_pack_kv_mixed: rec must be 16-byte aligned");
    return launched(csa::launch_pack_kv_mixed(x, x_dtype == CSA_BF16, rec, rows, static_cast<hipStream_t>(stream)),
                    "csa_pack_kv_mixed");
}

int csa_index_score_fp8(const unsigned char* q, const float* w, const unsigned char* k, const float* k_scale,
                        float* scores, int batch, int t, int h_i, int d_i, int n, const int* q_pos, int ratio,
                        long long q_stride_b, long long w_stride_b, long long k_stride_b, long long ks_stride_b,
                        long long s_stride_b, long long ld_s, csa_stream stream) {
    const int rc = check_fp8_score_args(q, w, k, k_scale, scores, batch, t, h_i, d_i, n, ratio, q_stride_b,
                                        w_stride_b, k_stride_b, ks_stride_b, s_stride_b, ld_s,
                                        "csa_index_score_fp8");
    if (rc != CSA_OK) return rc;
    csa::Fp8ScoreArgs a{q, w, k, k_scale, scores, batch, t, n, q_pos, ratio,
                        q_stride_b, w_stride_b, k_stride_b, ks_stride_b, s_stride_b, ld_s, csa::CandArgs{nullptr, 0, 0, 0}};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (t >= csa::kMqMinRows)
        return launched(csa::launch_index_score_mq_fp8(a, -1, s), "csa_index_score_fp8");
    return launched(csa::launch_index_score_fp8(a, nullptr, s), "csa_index_score_fp8");
}

int csa_index_score_fp4(const unsigned char* q, const float* w, const unsigned char* k, const unsigned int* k_scales,
                        float* scores, int batch, int t, int h_i, int d_i, int n, const int* q_pos, int ratio,
                        long long q_stride_b, long long w_stride_b, long long k_stride_b, long long ks_stride_b,
                        long long s_stride_b, long long ld_s, csa_stream stream) {
    const float* ks = reinterpret_cast<const float*>(k_scales);  // four E8M0 bytes per key (a 32-bit word)
    const int rc = check_fp8_score_args(q, w, k, ks, scores, batch, t, h_i, d_i, n, ratio, q_stride_b, w_stride_b,
                                        k_stride_b, ks_stride_b, s_stride_b, ld_s, "csa_index_score_fp4");
    if (rc != CSA_OK) return rc;
    csa::Fp8ScoreArgs a{q, w, k, ks, scores, batch, t, n, q_pos, ratio,
                        q_stride_b, w_stride_b, k_stride_b, ks_stride_b, s_stride_b, ld_s, csa::CandArgs{nullptr, 0, 0, 0}};
    a.k_fp4 = 1;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (t >= csa::kMqMinRows)
        return launched(csa::launch_index_score_mq_fp8(a, -1, s), "csa_index_score_fp4");
    return launched(csa::launch_index_score_fp8(a, nullptr, s), "csa_index_score_fp4");
}

size_t csa_topk_workspace_size(int batch, int t, int n, int k) {
    if (batch < 1 || t < 1 || n < 0 || k < 1) return 0;
    return csa::topk_workspace_bytes(batch * t, n, k);
}

int csa_topk(const float* scores, int batch, int t, int n, long long ld_s, long long s_stride_b,
             int k, int* idx, int* count, void* ws, size_t ws_bytes, csa_stream stream) {
    CHECK(idx && ws && (scores || n == 0), "csa_topk: null pointer argument");
    CHECK(batch >= 1 && t >= 1 && n >= 0, "csa_topk: batch %d t %d n %d", batch, t, n);
    CHECK(batch * static_cast<long long>(t) <= 65535, "csa_topk: batch*t above 65535");
    CHECK(k >= 1 && k <= csa::kTopkMaxK, "csa_topk: k=%d out of 1..%d", k, csa::kTopkMaxK);
    CHECK(ld_s >= n && s_stride_b >= 0, "csa_topk: bad strides");
    CHECK(aligned16(ws), "csa_topk: workspace must be 16-byte aligned");
    if (ws_bytes < csa_topk_workspace_size(batch, t, n, k))
        return fail(CSA_ERR_WORKSPACE, "csa_topk: workspace %zu < %zu bytes", ws_bytes,
                    csa_topk_workspace_size(batch, t, n, k));
    csa::TopkArgs a{scores, batch, t, n, ld_s, s_stride_b, k, idx, count, ws};
    return launched(csa::launch_topk(a, nullptr, static_cast<hipStream_t>(stream)), "csa_topk");
}

int csa_gather(const void* comp_kv, int n_comp, const int* idx, const int* count, int k,
               const void* swa, int swa_head, int swa_len, int w, void* gather_buf, int* n_valid,
               csa_dtype dtype, int batch, int d, long long kv_stride_b, long long swa_stride_b,
               long long buf_stride_b, csa_stream stream) {
    CHECK(gather_buf && (idx || k == 0) && (comp_kv || n_comp == 0) && (swa || swa_len == 0),
          "csa_gather: null pointer argument");
    CHECK(dtype_ok(dtype), "csa_gather: bad dtype");
    CHECK(batch >= 1 && d >= 1 && k >= 0 && n_comp >= 0, "csa_gather: bad sizes");
    CHECK(w >= 1 && swa_head >= 0 && swa_head < w && swa_len >= 0 && swa_len <= w,
          "csa_gather: bad window (w %d head %d len %d)", w, swa_head, swa_len);
    CHECK((static_cast<long long>(d) * elem_size(dtype)) % 16 == 0, "csa_gather: row bytes must be a multiple of 16");
    CHECK(aligned16(gather_buf) && (!comp_kv || aligned16(comp_kv)) && (!swa || aligned16(swa)),
          "csa_gather: buffers must be 16-byte aligned");
    CHECK(kv_stride_b >= 0 && swa_stride_b >= 0 && buf_stride_b >= 0, "csa_gather: negative stride");
    const int es = elem_size(dtype);
    CHECK((kv_stride_b * es) % 16 == 0 && (swa_stride_b * es) % 16 == 0 && (buf_stride_b * es) % 16 == 0,
          "csa_gather: batch strides must keep 16-byte alignment");
    return launched(csa::launch_gather(comp_kv, n_comp, idx, count, k, swa, swa_head, swa_len, w,
                                       gather_buf, n_valid, es, batch, d, kv_stride_b, swa_stride_b,
                                       buf_stride_b, static_cast<hipStream_t>(stream)),
                    "csa_gather");
}

size_t csa_sparse_attn_workspace_size(int batch, int h, int d, int n_max) {
    if (batch < 1 || h < 1 || d < 1 || n_max < 0) return 0;
    const size_t s = csa::attn_workspace_bytes(true, batch, h, d, n_max);
    return s > 0 ? s : 16;
}

static int check_attn(const void* q, const void* kv, const int* n_valid, void* out,
                      csa_dtype dtype, csa_dtype out_dtype, int batch, int h, int d, int n_max,
                      long long q_stride_b, long long kv_stride_b, long long out_stride_b,
                      const char* who) {
    CHECK(q && kv && n_valid && out, "%s: null pointer argument", who);
    CHECK(dtype_ok(dtype) && dtype_ok(out_dtype), "%s: bad dtype", who);
    CHECK(batch >= 1 && h >= 1 && d >= 1 && n_max >= 0, "%s: bad sizes", who);
    CHECK(q_stride_b >= 0 && kv_stride_b >= 0 && out_stride_b >= 0, "%s: negative stride", who);
    if (dtype == CSA_BF16) {
        if (h % 16 != 0 || d % 32 != 0 || d > 512 || n_max > csa::attn_max_rows())
            return fail(CSA_ERR_UNSUPPORTED, "%s: bf16 path needs h%%16==0, d%%32==0, d<=512, n_max<=%d", who,
                        csa::attn_max_rows());
        CHECK(aligned16(q) && aligned16(kv), "%s: q, kv must be 16-byte aligned", who);
        CHECK(q_stride_b % 8 == 0 && kv_stride_b % 8 == 0, "%s: batch strides must keep 16-byte alignment", who);
        CHECK(batch <= 65535 && h / 16 <= 65535, "%s: grid too large", who);
    } else {
        if (d > 1024 || n_max > 8192)
            return fail(CSA_ERR_UNSUPPORTED, "%s: f32 path needs d<=1024, n_max<=8192", who);
    }
    return CSA_OK;
}

int csa_sparse_attn(const void* q, const void* kv, const int* n_valid, const float* sink, float scale,
                    void* out, float* lse, csa_dtype dtype, csa_dtype out_dtype, int batch, int h,
                    int d, int n_max, long long q_stride_b, long long kv_stride_b,
                    long long out_stride_b, void* ws, size_t ws_bytes, csa_stream stream) {
    const int rc = check_attn(q, kv, n_valid, out, dtype, out_dtype, batch, h, d, n_max, q_stride_b,
                              kv_stride_b, out_stride_b, "csa_sparse_attn");
    if (rc != CSA_OK) return rc;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == CSA_BF16) {
        CHECK(ws && aligned16(ws), "csa_sparse_attn: workspace missing or misaligned");
        const size_t need = csa::attn_workspace_bytes(true, batch, h, d, n_max);
        if (ws_bytes < need)
            return fail(CSA_ERR_WORKSPACE, "csa_sparse_attn: workspace %zu < %zu bytes", ws_bytes, need);
        csa::AttnArgs a{};
        a.q = static_cast<const uint16_t*>(q);
        a.q_stride_b = q_stride_b;
        a.kv = static_cast<const uint16_t*>(kv);
        a.kv_stride_b = kv_stride_b;
        a.n_valid = n_valid;
        a.sink = sink;
        a.scale = scale;
        a.out = out;
        a.out_bf16 = out_dtype == CSA_BF16;
        a.lse = lse;
        a.out_stride_b = out_stride_b;
        a.batch = batch;
        a.h = h;
        a.d = d;
        a.n_max = n_max;
        a.ws = ws;
        return launched(csa::launch_attn_bf16(a, s), "csa_sparse_attn");
    }
    return launched(csa::launch_attn_f32(q, kv, n_valid, sink, scale, out, out_dtype == CSA_BF16, lse,
                                         batch, h, d, n_max, q_stride_b, kv_stride_b, out_stride_b, s),
                    "csa_sparse_attn");
}

// ---- fused decode step ------------------------------------------------------------

// Candidate slots reserved per sequence for the score kernel's top-k lists
// (the kernel uses two workgroups per compute unit; beyond this many the step
// falls back to the exact top-k path).
constexpr int kStepMaxSlots = 1024;
// rows short enough for every attention workgroup to take the exact top-k path itself
constexpr int kFuseExactMaxN = 8192;

static size_t step_topk_bytes(const csa_layer_desc* L) {
    return align256(static_cast<size_t>(L->batch) * kStepMaxSlots * csa::kMaxCandM1 * sizeof(unsigned long long));
}

// the two-stage E4M3 selection's list of exact candidates (one per sequence)
static size_t step_rescore_bytes(const csa_layer_desc* L) {
    if ((L->idx_dtype != CSA_FP8_E4M3 && L->idx_dtype != CSA_FP4_E2M1) || L->idx_rescore <= 0) return 0;
    return align256(static_cast<size_t>(L->batch) * (static_cast<size_t>(L->idx_rescore) + 1) *
                    sizeof(unsigned long long));
}

size_t csa_decode_step_workspace_size(const csa_layer_desc* L) {
    if (!L || L->batch < 1 || L->max_comp < 0 || L->top_k < 1) return 0;
    return step_topk_bytes(L) +
           align256(csa::attn_workspace_bytes(L->dtype == CSA_BF16, L->batch, L->h, L->d, L->top_k + L->w)) +
           256 + step_rescore_bytes(L);
}

size_t csa_decode_step_dev_ring_size(const csa_layer_desc* L) {
    if (!L || L->batch < 1 || L->m < 1 || L->d < 1 || L->d_i < 0) return 0;
    const size_t wm = static_cast<size_t>(L->overlap ? 2 * L->d : L->d);
    const size_t wi = static_cast<size_t>(L->overlap ? 2 * L->d_i : L->d_i);
    return sizeof(float) * static_cast<size_t>(L->batch) * 4 * L->m * (wm + wi);
}

// Which kernels of the step an entry point enqueues: all of them, or the
// first (jobs + scan) or the rest (top-k + gather + attention) of the
// two-call form.  Both calls validate everything and size every launch the
// same way, so their candidate slots agree.
enum StepPhase { kStepAll = 0, kStepScan = 1, kStepAttend = 2 };

// The decode step; dev != nullptr: the counters are read from and advanced
// on the device (csa_decode_step_dev), the block rows kept in `ring`.
static int decode_step(const csa_layer_desc* L, const csa_step_io* io, void* ws, size_t ws_bytes,
                       csa_stream stream, csa::DevState* dev, float* ring, size_t ring_bytes,
                       StepPhase phase = kStepAll) {
    CHECK(L && io, "csa_decode_step: null layer or io");
    CHECK(dtype_ok(L->dtype) && dtype_ok(L->out_dtype), "csa_decode_step: bad dtype");
    CHECK(L->batch >= 1 && L->m >= 1 && L->w >= 1 && L->top_k >= 1 && L->top_k <= csa::kTopkMaxK,
          "csa_decode_step: bad batch/m/w/top_k");
    CHECK(L->overlap == 0 || L->overlap == 1, "csa_decode_step: overlap must be 0 or 1");
    CHECK(L->comp_kv && L->idx_keys && L->swa && L->main_bias && L->idx_bias,
          "csa_decode_step: null cache or bias pointer");
    CHECK(io->q && io->q_idx && io->w_idx && io->kv_new && io->scores && io->topk_idx &&
              io->topk_count && io->gather_buf && io->n_valid && io->out,
          "csa_decode_step: null io pointer");
    if (dev) {
        // the counters live on the device; every step brings its token's Z/C rows
        CHECK(aligned16(dev), "csa_decode_step_dev: state must be 16-byte aligned");
        CHECK(io->z_main && io->c_main && io->z_idx && io->c_idx, "csa_decode_step_dev: Z/C rows missing");
        CHECK(ring && aligned16(ring), "csa_decode_step_dev: ring must be non-null and 16-byte aligned");
        CHECK(ring_bytes >= csa_decode_step_dev_ring_size(L), "csa_decode_step_dev: ring %zu < %zu bytes",
              ring_bytes, csa_decode_step_dev_ring_size(L));
        CHECK(L->max_comp >= 1, "csa_decode_step_dev: max_comp must be positive");
        if (L->dtype != CSA_BF16)
            return fail(CSA_ERR_UNSUPPORTED, "csa_decode_step_dev: bfloat16 caches only");
    } else {
        CHECK(io->pos >= 0, "csa_decode_step: pos < 0");
        CHECK(L->n_comp >= 0 && L->n_comp <= L->max_comp, "csa_decode_step: n_comp %d outside 0..max_comp %d",
              L->n_comp, L->max_comp);
        CHECK(L->swa_head >= 0 && L->swa_head < L->w && L->swa_len >= 0 && L->swa_len <= L->w,
              "csa_decode_step: bad SWA state");
    }
    // with device counters: the roles that may compress are launched, the
    // kernels decide; N is bounded by the cache capacity
    const bool completes = dev ? true : io->pos % L->m == L->m - 1;
    if (completes && !dev) {
        CHECK(io->z_main && io->c_main && io->z_idx && io->c_idx, "csa_decode_step: block rows missing");
        CHECK(L->n_comp < L->max_comp, "csa_decode_step: compressed cache full (max_comp %d)", L->max_comp);
    }
    if (!aligned16(ws)) return fail(CSA_ERR_INVALID_ARG, "csa_decode_step: workspace must be 16-byte aligned");
    if (ws_bytes < csa_decode_step_workspace_size(L))
        return fail(CSA_ERR_WORKSPACE, "csa_decode_step: workspace %zu < %zu bytes", ws_bytes,
                    csa_decode_step_workspace_size(L));
    const int N = dev ? L->max_comp : L->n_comp + (completes ? 1 : 0);
    // E4M3 or E2M1 indexer keys: bfloat16 everything else, the FP8 score
    // kernel (its E2M1 form for FP4 keys); below `fp8` covers both
    const bool fp4 = L->idx_dtype == CSA_FP4_E2M1;
    const bool fp8 = L->idx_dtype == CSA_FP8_E4M3 || fp4;
    if (fp8 && L->dtype != CSA_BF16)
        return fail(CSA_ERR_UNSUPPORTED, "csa_decode_step: E4M3 / E2M1 indexer keys need bfloat16 caches");
    // the two-stage E4M3 selection: the k_cand best by E4M3 score, rescored from bfloat16 keys
    const bool rescore = fp8 && L->idx_rescore > 0;
    if (L->idx_rescore != 0) {
        if (!fp8)
            return fail(CSA_ERR_UNSUPPORTED, "csa_decode_step: idx_rescore needs E4M3 or E2M1 indexer keys");
        if (dev)
            return fail(CSA_ERR_UNSUPPORTED, "csa_decode_step_dev: the two-stage E4M3 selection needs host counters");
        CHECK(L->idx_rescore >= L->top_k && L->idx_rescore <= csa::kTopkMaxK,
              "csa_decode_step: idx_rescore %d outside top_k %d .. %d", L->idx_rescore, L->top_k, csa::kTopkMaxK);
        CHECK(L->idx_keys_exact && aligned16(L->idx_keys_exact) && L->idx_keys_exact_stride_b % 8 == 0 &&
                  L->idx_keys_exact_stride_b >= 0,
              "csa_decode_step: idx_keys_exact missing, misaligned or with a bad batch stride");
    }
    const int kc = rescore ? L->idx_rescore : L->top_k;  // the first stage's k
    // (the E4M3 step takes a bfloat16 query and quantises it: its stride is in bfloat16 elements)
    const int rc_s = fp8 ? check_fp8_score_args(io->q_idx, io->w_idx, L->idx_keys, L->idx_scales, io->scores,
                                                L->batch, 1, L->h_i, L->d_i, N, L->m, 2 * io->q_idx_stride_b,
                                                io->w_stride_b, L->idx_keys_stride_b, L->idx_scales_stride_b,
                                                io->scores_stride_b, N, "csa_decode_step")
                         : check_score_args(io->q_idx, io->w_idx, L->idx_keys, io->scores, L->dtype, L->batch,
                                            1, L->h_i, L->d_i, N, L->m, io->q_idx_stride_b, io->w_stride_b,
                                            L->idx_keys_stride_b, io->scores_stride_b, N, "csa_decode_step");
    if (rc_s != CSA_OK) return rc_s;
    const int n_max = L->top_k + L->w;
    const int rc_a = check_attn(io->q, io->gather_buf, io->n_valid, io->out, L->dtype, L->out_dtype,
                                L->batch, L->h, L->d, n_max, io->q_stride_b, io->gather_stride_b,
                                io->out_stride_b, "csa_decode_step");
    if (rc_a != CSA_OK) return rc_a;
    const int es = elem_size(L->dtype);
    CHECK((static_cast<long long>(L->d) * es) % 16 == 0, "csa_decode_step: row bytes must be a multiple of 16");
    // mixed main KV: 592-byte records (mixed_kv.h), RoPE tables
    const bool mixed = L->kv_dtype == CSA_FP8_E4M3;
    if (mixed) {
        if (L->dtype != CSA_BF16 || L->d != csa::kMixD || L->rope_dim != csa::kMixRope)
            return fail(CSA_ERR_UNSUPPORTED, "csa_decode_step: mixed KV needs bfloat16, d = %d, rope_dim = %d",
                        csa::kMixD, csa::kMixRope);
        CHECK(L->rope_cos && L->rope_sin && L->comp_rope_cos && L->comp_rope_sin,
              "csa_decode_step: mixed KV needs both RoPE tables");
        CHECK(L->rope_rows >= 1 && L->comp_rope_rows >= 1, "csa_decode_step: empty RoPE table");
        CHECK(dev || io->pos < L->rope_rows, "csa_decode_step: pos %d outside the RoPE table (%d rows)", io->pos,
              L->rope_rows);
        CHECK(dev || !completes || io->pos / L->m < L->comp_rope_rows,
              "csa_decode_step: block %d outside the compressed-entry RoPE table (%d rows)", io->pos / L->m,
              L->comp_rope_rows);
        CHECK(aligned16(L->comp_kv) && aligned16(L->swa) && aligned16(io->gather_buf) &&
                  L->comp_kv_stride_b % 16 == 0 && L->swa_stride_b % 16 == 0 && io->gather_stride_b % 16 == 0,
              "csa_decode_step: mixed records and their batch strides must be 16-byte aligned");
    }

    CHECK(L->d <= csa::kPrepMaxD && L->d_i <= csa::kPrepMaxD, "csa_decode_step: head dims above %d", csa::kPrepMaxD);
    CHECK((static_cast<long long>(L->d_i) * es) % 16 == 0 || !completes, "csa_decode_step: d_i row bytes must be a multiple of 16");

    const hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf = L->dtype == CSA_BF16;
    hipError_t e;
    void* tws = ws;
    void* aws = static_cast<char*>(ws) + step_topk_bytes(L);
    const int swa_head = (L->swa_head + 1) % L->w;
    const int swa_len = L->swa_len + 1 < L->w ? L->swa_len + 1 : L->w;

    // a+b. SWA append and compression of the completed block
    csa::PrepArgs pa{};
    pa.batch = L->batch;
    pa.es = es;
    pa.d = L->d;
    pa.d_i = L->d_i;
    pa.m = L->m;
    pa.overlap = L->overlap;
    pa.completes = completes ? 1 : 0;
    pa.n_comp = dev ? 0 : L->n_comp;
    pa.block = dev ? 0 : io->pos / L->m;
    pa.kv_new = io->kv_new;
    pa.kv_new_stride_b = io->kv_new_stride_b;
    pa.swa = L->swa;
    pa.swa_stride_b = L->swa_stride_b;
    pa.swa_slot = L->swa_head;
    if (completes && !dev) {
        // the overlapped form passes the previous block's rows first
        const bool joint = L->overlap && io->pos / L->m > 0;
        const long long skip_main = joint ? static_cast<long long>(L->m) * 2 * L->d : 0;
        const long long skip_idx = joint ? static_cast<long long>(L->m) * 2 * L->d_i : 0;
        pa.z_main = io->z_main + skip_main;
        pa.c_main = io->c_main + skip_main;
        pa.z_idx = io->z_idx + skip_idx;
        pa.c_idx = io->c_idx + skip_idx;
    }
    pa.zc_main_stride_b = io->zc_main_stride_b;
    pa.zc_idx_stride_b = io->zc_idx_stride_b;
    pa.main_bias = L->main_bias;
    pa.idx_bias = L->idx_bias;
    pa.main_norm = L->main_norm;
    pa.idx_norm = L->idx_norm;
    pa.comp_kv = L->comp_kv;
    pa.comp_kv_stride_b = L->comp_kv_stride_b;
    pa.idx_keys = L->idx_keys;
    pa.idx_keys_stride_b = L->idx_keys_stride_b;
    pa.idx_fp8 = fp8 ? 1 : 0;
    pa.idx_fp4 = fp4 ? 1 : 0;
    pa.idx_scales = fp8 ? L->idx_scales : nullptr;
    pa.idx_scales_stride_b = fp8 ? L->idx_scales_stride_b : 0;
    pa.idx_keys_exact = rescore ? static_cast<uint16_t*>(L->idx_keys_exact) : nullptr;
    pa.idx_keys_exact_stride_b = rescore ? L->idx_keys_exact_stride_b : 0;
    if (dev) {  // the token's own rows; the kernels keep the block in the ring
        pa.z_main = io->z_main;
        pa.c_main = io->c_main;
        pa.z_idx = io->z_idx;
        pa.c_idx = io->c_idx;
        pa.dev = dev;
        pa.max_comp = L->max_comp;
        pa.swa_w = L->w;
        pa.dev_ring = ring;
        pa.ring_stride_b = static_cast<long long>(csa_decode_step_dev_ring_size(L) / sizeof(float) / L->batch);
        pa.comp_rope_cos = L->comp_rope_cos;
        pa.comp_rope_sin = L->comp_rope_sin;
        pa.comp_rope_rows = L->comp_rope_rows;
    }
    pa.kv_mixed = mixed ? 1 : 0;
    if (mixed && completes && !dev) {
        const long long row = static_cast<long long>(io->pos / L->m) * (csa::kMixRope / 2);
        pa.entry_cos = L->comp_rope_cos + row;
        pa.entry_sin = L->comp_rope_sin + row;
    }
    // The bf16 and E4M3 score kernels runs these jobs in its first workgroups (and
    // scores the new key itself); the float32 path launches them first.
    const int n_scan = dev ? L->max_comp : (bf ? L->n_comp : N);
    const int prep_wgs = bf ? (completes ? 3 : 1) : 0;
    const bool do_scan = phase != kStepAttend;
    const bool do_rest = phase != kStepScan;
    if (!bf && do_scan) {
        e = csa::launch_step_prep(pa, s);
        if (e != hipSuccess) return launched(e, "csa_decode_step/prep");
    }

    // c. score, with every workgroup's top-k candidates when the rows are long,
    //    then the exact top-k
    csa::CandArgs ca{nullptr, 0, 0, 0};
    if (bf && N > 0) {
        const int slots = (fp8 ? csa::index_score_fp8_wgs(L->batch, n_scan, prep_wgs)
                               : csa::index_score_bf16_wgs(L->batch, n_scan, prep_wgs)) +
                          (completes ? 1 : 0);
        const int kpw = fp8 ? csa::index_score_fp8_keys_per_wg(L->batch, n_scan, prep_wgs)
                            : csa::index_score_bf16_keys_per_wg(L->batch, n_scan, prep_wgs);
        const int m = kpw > 0 ? csa::topk_cand_m(N, kc, kpw) : -1;
        const int mw = kpw > 0 ? csa::topk_cand_m(N, kc, kpw / csa::kScoreWavesPerWg) : -1;
        // a scan workgroup's waves take consecutive 16-key tiles, the grid strides over the row
        const int run = csa::kScoreWavesPerWg * 16;
        const int scan_wgs = slots - (completes ? 1 : 0);
        if (m > 0 && slots <= kStepMaxSlots && (dev || N > 4 * kc))
            ca = csa::CandArgs{static_cast<unsigned long long*>(tws), slots, m, mw < m ? mw : m, run, scan_wgs * run};
    }
    csa::ScoreArgs sa{io->q_idx, io->w_idx, L->idx_keys, io->scores, L->batch, 1, L->h_i, L->d_i, n_scan,
                      nullptr, L->m, io->q_idx_stride_b, io->w_stride_b, L->idx_keys_stride_b,
                      io->scores_stride_b, N, ca, dev};
    if (!do_scan) {
        e = hipSuccess;
    } else if (fp8) {
        const csa::Fp8ScoreArgs fa{static_cast<const uint8_t*>(io->q_idx), io->w_idx,
                                   static_cast<const uint8_t*>(L->idx_keys), L->idx_scales, io->scores,
                                   L->batch, 1, n_scan, nullptr, L->m, 2 * io->q_idx_stride_b, io->w_stride_b,
                                   L->idx_keys_stride_b, L->idx_scales_stride_b, io->scores_stride_b, N, ca, dev,
                                   static_cast<const uint16_t*>(io->q_idx), io->q_idx_stride_b, fp4 ? 1 : 0};
        e = csa::launch_index_score_fp8(fa, &pa, s);
    } else {
        e = bf ? csa::launch_index_score_bf16(sa, &pa, s) : csa::launch_index_score_f32(sa, s);
    }
    if (e != hipSuccess) return launched(e, "csa_decode_step/index_score");
    if (!do_rest) return ok();
    csa::TopkArgs ta{io->scores, L->batch, 1, N, N, io->scores_stride_b, L->top_k, io->topk_idx,
                     io->topk_count, tws};
    if (dev) {
        ta.dev = dev;
        ta.w = L->w;
        ta.m = L->m;
        ta.max_comp = L->max_comp;
    }
    // two-stage E4M3 selection: the first stage and the exact scores make one
    // list per sequence that the top-k below selects from
    if (rescore) {
        auto* ex = reinterpret_cast<unsigned long long*>(
            static_cast<char*>(ws) + csa_decode_step_workspace_size(L) - step_rescore_bytes(L));
        csa::TopkArgs tc = ta;
        tc.k = kc;
        const csa::RescoreArgs ra{static_cast<const uint16_t*>(io->q_idx), io->q_idx_stride_b, io->w_idx,
                                  io->w_stride_b, static_cast<const uint16_t*>(L->idx_keys_exact),
                                  L->idx_keys_exact_stride_b, N, ex};
        e = csa::launch_fp8_rescore(tc, ca.lists ? &ca : nullptr, ra, s);
        if (e != hipSuccess) return launched(e, "csa_decode_step/rescore");
        ca = csa::CandArgs{ex, 1, kc, kc};
    }
    // bf16 with candidate lists (or a short row): every attention workgroup
    // selects the top k itself, no separate top-k launch, as long as those
    // workgroups are all resident at once (one per compute unit); a larger batch
    // selects once per sequence and attends with smaller workgroups.  The
    // device-counter step takes the separate launches only with candidate
    // lists (its entry count is on the device: without lists the top-k must
    // read the whole row, which the fused kernel bounds by that count).
    const bool all_resident = csa::topk_attn_workgroups(L->batch, L->h, n_max) <= csa::device_cu_count();
    const bool fuse = bf && (dev ? (!ca.lists || all_resident)
                                 : ((ca.lists || N <= kFuseExactMaxN) && all_resident));
    if (!fuse) {
        e = csa::launch_topk(ta, ca.lists ? &ca : nullptr, s);
        if (e != hipSuccess) return launched(e, "csa_decode_step/topk");
    }

    // d+e. gather (fused into the attention on the bf16 path) and attention
    if (bf) {
        csa::AttnArgs a{};
        a.q = static_cast<const uint16_t*>(io->q);
        a.q_stride_b = io->q_stride_b;
        a.comp_kv = static_cast<const uint16_t*>(L->comp_kv);
        a.comp_kv_stride_b = L->comp_kv_stride_b;
        a.n_comp = N;
        a.idx = io->topk_idx;
        a.count = io->topk_count;
        a.k = L->top_k;
        a.swa = static_cast<const uint16_t*>(L->swa);
        a.swa_stride_b = L->swa_stride_b;
        a.swa_head = swa_head;
        a.swa_len = swa_len;
        a.w = L->w;
        a.gather_buf = static_cast<uint16_t*>(io->gather_buf);
        a.buf_stride_b = io->gather_stride_b;
        a.n_valid_out = io->n_valid;
        a.sink = L->sink;
        a.scale = L->scale;
        a.out = io->out;
        a.out_bf16 = L->out_dtype == CSA_BF16;
        a.lse = io->lse;
        a.out_stride_b = io->out_stride_b;
        a.batch = L->batch;
        a.h = L->h;
        a.d = L->d;
        a.n_max = n_max;
        a.ws = aws;
        if (mixed) {
            a.kv_mixed = true;
            if (!dev) {
                const long long row = static_cast<long long>(io->pos) * (csa::kMixRope / 2);
                a.inv_cos = L->rope_cos + row;
                a.inv_sin = L->rope_sin + row;
            }
        }
        if (dev) {
            a.dev = dev;
            a.m = L->m;
            a.max_comp = L->max_comp;
            a.rope_cos = L->rope_cos;
            a.rope_sin = L->rope_sin;
            a.rope_rows = L->rope_rows;
            // one int past the attention workspace (inside the step's slack)
            a.dev_pos = reinterpret_cast<int*>(static_cast<char*>(aws) +
                                               align256(csa::attn_workspace_bytes(true, L->batch, L->h, L->d, n_max)));
            a.dev_adv = dev;
        }
        e = fuse ? csa::launch_topk_attn(ta, ca.lists ? &ca : nullptr, a, s) : csa::launch_attn_bf16(a, s);
        return launched(e, "csa_decode_step/attention");
    }
    e = csa::launch_gather(L->comp_kv, N, io->topk_idx, io->topk_count, L->top_k, L->swa, swa_head,
                           swa_len, L->w, io->gather_buf, io->n_valid, es, L->batch, L->d,
                           L->comp_kv_stride_b, L->swa_stride_b, io->gather_stride_b, s);
    if (e != hipSuccess) return launched(e, "csa_decode_step/gather");
    e = csa::launch_attn_f32(io->q, io->gather_buf, io->n_valid, L->sink, L->scale, io->out,
                             L->out_dtype == CSA_BF16, io->lse, L->batch, L->h, L->d, n_max,
                             io->q_stride_b, io->gather_stride_b, io->out_stride_b, s);
    return launched(e, "csa_decode_step/attention");
}

int csa_decode_step(const csa_layer_desc* L, const csa_step_io* io, void* ws, size_t ws_bytes,
                    csa_stream stream) {
    return decode_step(L, io, ws, ws_bytes, stream, nullptr, nullptr, 0);
}

int csa_decode_step_scan(const csa_layer_desc* L, const csa_step_io* io, void* ws, size_t ws_bytes,
                         csa_stream stream) {
    return decode_step(L, io, ws, ws_bytes, stream, nullptr, nullptr, 0, kStepScan);
}

int csa_decode_step_attend(const csa_layer_desc* L, const csa_step_io* io, void* ws, size_t ws_bytes,
                           csa_stream stream) {
    return decode_step(L, io, ws, ws_bytes, stream, nullptr, nullptr, 0, kStepAttend);
}

}  // extern "C"

// ---- the decode step without a caller workspace ----------------------------------------
//
// For callers that cannot allocate (graph capture, serving loops): the
// step's scratch (candidate lists, split partials) lives in this file-scope
// device array, one copy per GPU, held until the process ends.  On the host
// the array's name is only a stand-in: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is handed to
// kernels.  Nothing in the array has to start at zero: every byte the step
// reads back is written by the same step first.
namespace {

constexpr size_t kNoAllocScratchBytes = size_t{32} << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (nullptr and a message on failure).
void* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        fail(CSA_ERR_LAUNCH, "csa_decode_step_noalloc: no current device (or device id %d above %d)", dev,
             kMaxDevices - 1);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            fail(CSA_ERR_LAUNCH, "csa_decode_step_noalloc: hipGetSymbolAddress(scratch) failed: %s",
                 hipGetErrorString(e));
            return nullptr;
        }
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t csa_decode_step_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

int csa_decode_step_noalloc(const csa_layer_desc* L, const csa_step_io* io, csa_stream stream) {
    CHECK(L && io, "csa_decode_step_noalloc: null layer or io");
    const size_t need = csa_decode_step_workspace_size(L);
    CHECK(need > 0, "csa_decode_step_noalloc: bad layer sizes");
    if (need > kNoAllocScratchBytes)
        return fail(CSA_ERR_WORKSPACE,
                    "csa_decode_step_noalloc: the step needs %zu bytes of scratch, above the fixed %zu "
                    "(use csa_decode_step with a workspace)",
                    need, kNoAllocScratchBytes);
    void* ws = device_scratch();
    if (!ws) return CSA_ERR_LAUNCH;
    return decode_step(L, io, ws, kNoAllocScratchBytes, stream, nullptr, nullptr, 0);
}

int csa_decode_step_dev(const csa_layer_desc* L, const csa_step_io* io, csa_dev_state* state, float* ring,
                        size_t ring_bytes, void* ws, size_t ws_bytes, csa_stream stream) {
    static_assert(sizeof(csa_dev_state) == sizeof(csa::DevState), "device counters as the kernels read them");
    CHECK(state, "csa_decode_step_dev: null state");
    return decode_step(L, io, ws, ws_bytes, stream, reinterpret_cast<csa::DevState*>(state), ring, ring_bytes);
}

size_t csa_hca_decode_step_workspace_size(const csa_layer_desc* L) {
    if (!L || L->batch < 1 || L->max_comp < 0 || L->w < 1 || L->h < 1 || L->d < 1) return 0;
    const size_t ns = static_cast<size_t>(csa::attn_dense_splits(L->max_comp + L->w));
    // split partials, then (mixed KV) the new entry in float32 per sequence,
    // then (device counters) the step's record for the merge
    return align256(sizeof(float) * static_cast<size_t>(L->batch) * L->h * ns * (static_cast<size_t>(L->d) + 2)) +
           align256(sizeof(float) * static_cast<size_t>(L->batch) * L->d) + 256 + 256;
}

size_t csa_hca_decode_step_dev_ring_size(const csa_layer_desc* L) {
    if (!L || L->batch < 1 || L->m < 1 || L->d < 1) return 0;
    return sizeof(float) * static_cast<size_t>(L->batch) * 4 * L->m * static_cast<size_t>(L->d);
}

// The HCA step; dev != nullptr: the counters are read from and advanced on
// the device (csa_hca_decode_step_dev), the block's rows kept in `ring`.
static int hca_step(const csa_layer_desc* L, const csa_step_io* io, void* ws, size_t ws_bytes, csa_stream stream,
                    csa::DevState* dev, float* ring, size_t ring_bytes) {
    const char* who = dev ? "csa_hca_decode_step_dev" : "csa_hca_decode_step";
    CHECK(L && io, "%s: null layer or io", who);
    if (L->dtype != CSA_BF16)
        return fail(CSA_ERR_UNSUPPORTED, "%s: bfloat16 caches only", who);
    const bool mixed = L->kv_dtype == CSA_FP8_E4M3;
    if (mixed) {
        if (L->d != csa::kMixD || L->rope_dim != csa::kMixRope || L->main_norm)
            return fail(CSA_ERR_UNSUPPORTED, "%s: mixed KV needs d = %d, rope_dim = %d, no main norm", who,
                        csa::kMixD, csa::kMixRope);
        CHECK(L->rope_cos && L->rope_sin && L->comp_rope_cos && L->comp_rope_sin && L->rope_rows >= 1 &&
                  L->comp_rope_rows >= 1,
              "%s: mixed KV needs both RoPE tables", who);
        CHECK(dev || io->pos < L->rope_rows, "%s: pos %d outside the RoPE table (%d rows)", who, io->pos,
              L->rope_rows);
        CHECK(dev || io->pos % L->m != L->m - 1 || io->pos / L->m < L->comp_rope_rows,
              "%s: block %d outside the compressed-entry RoPE table (%d rows)", who, io->pos / L->m,
              L->comp_rope_rows);
        CHECK(L->comp_kv_stride_b % 16 == 0 && L->swa_stride_b % 16 == 0,
              "%s: mixed records' batch strides must be multiples of 16 bytes", who);
    }
    CHECK(dtype_ok(L->out_dtype), "%s: bad out_dtype", who);
    CHECK(L->batch >= 1 && L->m >= 1 && L->w >= 1, "%s: bad batch/m/w", who);
    CHECK(L->overlap == 0, "%s: the HCA compressor is not overlapped (overlap must be 0)", who);
    CHECK(L->comp_kv && L->swa && L->main_bias, "%s: null cache or bias pointer", who);
    CHECK(io->q && io->kv_new && io->out, "%s: null io pointer", who);
    if (dev) {
        CHECK(aligned16(dev), "%s: state must be 16-byte aligned", who);
        CHECK(io->z_main && io->c_main, "%s: the token's Z/C rows missing", who);
        CHECK(ring && aligned16(ring), "%s: ring must be non-null and 16-byte aligned", who);
        CHECK(ring_bytes >= csa_hca_decode_step_dev_ring_size(L), "%s: ring %zu < %zu bytes", who, ring_bytes,
              csa_hca_decode_step_dev_ring_size(L));
        CHECK(L->max_comp >= 1, "%s: max_comp must be positive", who);
    } else {
        CHECK(io->pos >= 0, "%s: pos < 0", who);
        CHECK(L->n_comp >= 0 && L->n_comp <= L->max_comp, "%s: n_comp %d outside 0..max_comp %d", who, L->n_comp,
              L->max_comp);
        CHECK(L->swa_head >= 0 && L->swa_head < L->w && L->swa_len >= 0 && L->swa_len <= L->w,
              "%s: bad SWA state", who);
    }
    // with device counters the launch is shaped for a completing step; the kernels decide
    const bool completes = dev ? true : io->pos % L->m == L->m - 1;
    if (completes && !dev) {
        CHECK(io->z_main && io->c_main, "%s: block rows missing", who);
        CHECK(L->n_comp < L->max_comp, "%s: compressed cache full (max_comp %d)", who, L->max_comp);
    }
    const int n_max = L->max_comp + L->w;
    if (n_max > csa::attn_max_rows())
        return fail(CSA_ERR_UNSUPPORTED, "%s: max_comp + w = %d above %d rows", who, n_max, csa::attn_max_rows());
    CHECK(L->h >= 16 && L->h % 16 == 0 && L->d >= 32 && L->d % 32 == 0 && L->d <= 512,
          "%s: needs h a multiple of 16 and d a multiple of 32 up to 512", who);
    CHECK(L->d <= csa::kPrepMaxD, "%s: head dim above %d", who, csa::kPrepMaxD);
    CHECK(aligned16(io->q) && aligned16(L->comp_kv) && aligned16(L->swa) && aligned16(io->kv_new) &&
              aligned16(io->out),
          "%s: q, caches, kv_new and out must be 16-byte aligned", who);
    CHECK(io->q_stride_b % 8 == 0 && L->comp_kv_stride_b % 8 == 0 && L->swa_stride_b % 8 == 0 &&
              io->kv_new_stride_b % 8 == 0,
          "%s: batch strides must keep 16-byte alignment", who);
    if (!aligned16(ws)) return fail(CSA_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", who);
    if (ws_bytes < csa_hca_decode_step_workspace_size(L))
        return fail(CSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", who, ws_bytes,
                    csa_hca_decode_step_workspace_size(L));
    const hipStream_t s = static_cast<hipStream_t>(stream);

    // a+b. SWA append and (on completion) the main compressor; no indexer key
    csa::PrepArgs pa{};
    pa.batch = L->batch;
    pa.es = 2;
    pa.d = L->d;
    pa.m = L->m;
    pa.completes = completes ? 1 : 0;
    pa.n_comp = dev ? 0 : L->n_comp;
    pa.block = dev ? 0 : io->pos / L->m;
    pa.kv_new = io->kv_new;
    pa.kv_new_stride_b = io->kv_new_stride_b;
    pa.swa = L->swa;
    pa.swa_stride_b = L->swa_stride_b;
    pa.swa_slot = L->swa_head;
    pa.z_main = io->z_main;
    pa.c_main = io->c_main;
    pa.zc_main_stride_b = io->zc_main_stride_b;
    pa.main_bias = L->main_bias;
    pa.main_norm = L->main_norm;
    pa.comp_kv = L->comp_kv;
    pa.comp_kv_stride_b = L->comp_kv_stride_b;
    pa.idx_keys = nullptr;
    // long blocks without a norm: channel slices over several workgroups
    pa.main_wgs = (L->m >= 32 && !L->main_norm) ? (L->d + 31) / 32 : 1;
    pa.kv_mixed = mixed ? 1 : 0;
    if (mixed && completes && !dev) {
        const long long row = static_cast<long long>(io->pos / L->m) * (csa::kMixRope / 2);
        pa.entry_cos = L->comp_rope_cos + row;
        pa.entry_sin = L->comp_rope_sin + row;
    }
    if (dev) {  // the token's own rows; the kernels keep the block in the ring
        pa.dev = dev;
        pa.max_comp = L->max_comp;
        pa.swa_w = L->w;
        pa.dev_ring = ring;
        pa.ring_stride_b = static_cast<long long>(csa_hca_decode_step_dev_ring_size(L) / sizeof(float) / L->batch);
        pa.comp_rope_cos = L->comp_rope_cos;
        pa.comp_rope_sin = L->comp_rope_sin;
        pa.comp_rope_rows = L->comp_rope_rows;
    }

    // c. attention over the rows before the step — the entries before it and
    //    the window rows that stay (the new token's slot is being written) —
    //    in the same launch as a+b; the merge adds the new entry and token
    csa::AttnArgs a{};
    a.q = static_cast<const uint16_t*>(io->q);
    a.q_stride_b = io->q_stride_b;
    a.comp_kv = static_cast<const uint16_t*>(L->comp_kv);
    a.comp_kv_stride_b = L->comp_kv_stride_b;
    a.n_comp = dev ? 0 : L->n_comp;
    a.dense = true;
    a.swa = static_cast<const uint16_t*>(L->swa);
    a.swa_stride_b = L->swa_stride_b;
    a.swa_head = dev ? 0 : L->swa_head;
    a.swa_len = dev ? 0 : (L->swa_len + 1 < L->w ? L->swa_len + 1 : L->w) - 1;
    a.w = L->w;
    a.n_valid_out = io->n_valid;
    a.sink = L->sink;
    a.scale = L->scale;
    a.out = io->out;
    a.out_bf16 = L->out_dtype == CSA_BF16;
    a.lse = io->lse;
    a.out_stride_b = io->out_stride_b;
    a.batch = L->batch;
    a.h = L->h;
    a.d = L->d;
    a.n_max = n_max;
    a.ws = ws;
    if (mixed) {
        a.kv_mixed = true;
        if (!dev) {
            const long long row = static_cast<long long>(io->pos) * (csa::kMixRope / 2);
            a.inv_cos = L->rope_cos + row;
            a.inv_sin = L->rope_sin + row;
        }
    }
    if (dev) {
        a.dev = dev;
        a.m = L->m;
        a.max_comp = L->max_comp;
        a.rope_cos = L->rope_cos;
        a.rope_sin = L->rope_sin;
        a.rope_rows = L->rope_rows;
        a.comp_rope_cos = L->comp_rope_cos;
        a.comp_rope_sin = L->comp_rope_sin;
        a.comp_rope_rows = L->comp_rope_rows;
        // the step's record, in the last 256 bytes of the workspace
        a.dev_pos = reinterpret_cast<int*>(static_cast<char*>(ws) + csa_hca_decode_step_workspace_size(L) - 256);
        a.dev_adv = dev;
    }
    const void* x0 = completes && !mixed && !dev
                         ? static_cast<const char*>(L->comp_kv) + 2 * static_cast<long long>(L->n_comp) * L->d
                         : nullptr;
    return launched(csa::launch_attn_dense_bf16(a, pa, x0, L->comp_kv_stride_b, io->kv_new, io->kv_new_stride_b, s),
                    who);
}

int csa_hca_decode_step(const csa_layer_desc* L, const csa_step_io* io, void* ws, size_t ws_bytes,
                        csa_stream stream) {
    return hca_step(L, io, ws, ws_bytes, stream, nullptr, nullptr, 0);
}

int csa_hca_decode_step_dev(const csa_layer_desc* L, const csa_step_io* io, csa_dev_state* state, float* ring,
                            size_t ring_bytes, void* ws, size_t ws_bytes, csa_stream stream) {
    CHECK(state, "csa_hca_decode_step_dev: null state");
    return hca_step(L, io, ws, ws_bytes, stream, reinterpret_cast<csa::DevState*>(state), ring, ring_bytes);
}

int csa_layer_advance(csa_layer_desc* L, int pos) {
    CHECK(L && L->w >= 1 && L->m >= 1 && pos >= 0, "csa_layer_advance: bad arguments");
    if (pos % L->m == L->m - 1) {
        CHECK(L->n_comp < L->max_comp, "csa_layer_advance: compressed cache full");
        L->n_comp += 1;
    }
    L->swa_head = (L->swa_head + 1) % L->w;
    L->swa_len = L->swa_len + 1 < L->w ? L->swa_len + 1 : L->w;
    return ok();
}

size_t csa_index_topk_workspace_size(int t, int n, int top_k) {
    if (t < 1 || n < 0 || top_k < 1) return 0;
    return csa::index_topk_workspace_bytes(t, n, top_k);
}

int csa_index_topk(const void* q, const float* w, const void* k, int t, int h_i, int d_i, int n,
                   long long pos0, int ratio, int top_k, int* idx, int* count, void* ws, size_t ws_bytes,
                   csa_stream stream) {
    CHECK(q && w && idx && ws && (k || n == 0), "csa_index_topk: null pointer argument");
    CHECK(t >= 1 && n >= 0, "csa_index_topk: t %d n %d", t, n);
    CHECK(ratio >= 1, "csa_index_topk: ratio %d", ratio);
    CHECK(top_k >= 1 && top_k <= csa::kTopkMaxK, "csa_index_topk: top_k=%d out of 1..%d", top_k, csa::kTopkMaxK);
    if (h_i != 64 || d_i != 128)
        return fail(CSA_ERR_UNSUPPORTED, "csa_index_topk: needs h_i=64, d_i=128 (got %d, %d)", h_i, d_i);
    CHECK(aligned16(q) && aligned16(w) && aligned16(ws) && (n == 0 || aligned16(k)),
          "csa_index_topk: q, w, k and ws must be 16-byte aligned");
    if (ws_bytes < csa_index_topk_workspace_size(t, n, top_k))
        return fail(CSA_ERR_WORKSPACE, "csa_index_topk: workspace %zu < %zu bytes", ws_bytes,
                    csa_index_topk_workspace_size(t, n, top_k));
    csa::IndexTopkArgs a{static_cast<const uint16_t*>(q), w, static_cast<const uint16_t*>(k), t, n, pos0, ratio,
                         top_k, idx, count, ws};
    return launched(csa::launch_index_topk(a, static_cast<hipStream_t>(stream)), "csa_index_topk");
}

// csa_index_topk_fp8 and csa_index_topk_fp4: E4M3 query codes against E4M3
// keys with row scales, or E2M1 keys with E8M0 block scales (fp4)
static int index_topk_lowp(const unsigned char* q, const float* w, const unsigned char* k, const float* k_scale,
                           bool fp4, int t, int h_i, int d_i, int n, long long pos0, int ratio, int top_k, int* idx,
                           int* count, void* ws, size_t ws_bytes, csa_stream stream, const char* who) {
    CHECK(q && w && idx && ws && ((k && k_scale) || n == 0), "%s: null pointer argument", who);
    CHECK(t >= 1 && n >= 0, "%s: t %d n %d", who, t, n);
    CHECK(ratio >= 1, "%s: ratio %d", who, ratio);
    CHECK(top_k >= 1 && top_k <= csa::kTopkMaxK, "%s: top_k=%d out of 1..%d", who, top_k, csa::kTopkMaxK);
    if (h_i != 64 || d_i != 128)
        return fail(CSA_ERR_UNSUPPORTED, "%s: needs h_i=64, d_i=128 (got %d, %d)", who, h_i, d_i);
    CHECK(aligned16(q) && aligned16(w) && aligned16(ws) && (n == 0 || aligned16(k)),
          "%s: q, w, k and ws must be 16-byte aligned", who);
    if (ws_bytes < csa_index_topk_workspace_size(t, n, top_k))
        return fail(CSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", who, ws_bytes,
                    csa_index_topk_workspace_size(t, n, top_k));
    csa::IndexTopkArgs a{};
    a.w = w;
    a.t = t;
    a.n = n;
    a.pos0 = pos0;
    a.ratio = ratio;
    a.top_k = top_k;
    a.idx = idx;
    a.count = count;
    a.ws = ws;
    a.q8 = q;
    a.k8 = k;
    // a non-null scale pointer selects the low-precision scan (no key is read when n = 0)
    static const float kNoKeys = 1.f;
    a.k_scale = n > 0 ? k_scale : &kNoKeys;
    a.k_fp4 = fp4 ? 1 : 0;
    return launched(csa::launch_index_topk(a, static_cast<hipStream_t>(stream)), who);
}

int csa_index_topk_fp8(const unsigned char* q, const float* w, const unsigned char* k, const float* k_scale, int t,
                       int h_i, int d_i, int n, long long pos0, int ratio, int top_k, int* idx, int* count,
                       void* ws, size_t ws_bytes, csa_stream stream) {
    return index_topk_lowp(q, w, k, k_scale, false, t, h_i, d_i, n, pos0, ratio, top_k, idx, count, ws, ws_bytes,
                           stream, "csa_index_topk_fp8");
}

int csa_index_topk_fp4(const unsigned char* q, const float* w, const unsigned char* k, const unsigned int* k_scales,
                       int t, int h_i, int d_i, int n, long long pos0, int ratio, int top_k, int* idx, int* count,
                       void* ws, size_t ws_bytes, csa_stream stream) {
    return index_topk_lowp(q, w, k, reinterpret_cast<const float*>(k_scales), true, t, h_i, d_i, n, pos0, ratio,
                           top_k, idx, count, ws, ws_bytes, stream, "csa_index_topk_fp4");
}

// workspace of the two-stage E4M3 selection of a chunk: query codes, folded
// weights, the first stage's candidates and counts, then csa_index_topk's
static size_t rescored_parts(int t, int n, int k_cand, size_t* off) {
    const size_t tt = static_cast<size_t>(t);
    off[0] = 0;                                                      // codes [t][64][128]
    off[1] = off[0] + align256(tt * 64 * 128);                       // folded w [t][64]
    off[2] = off[1] + align256(tt * 64 * sizeof(float));             // candidates [t][k_cand]
    off[3] = off[2] + align256(tt * static_cast<size_t>(k_cand) * sizeof(int));  // counts [t]
    off[4] = off[3] + align256(tt * sizeof(int));                    // the first stage's workspace
    return off[4] + csa::index_topk_workspace_bytes(t, n, k_cand);
}

size_t csa_index_topk_fp8_rescored_workspace_size(int t, int n, int top_k, int k_cand) {
    if (t < 1 || n < 0 || top_k < 1 || k_cand < top_k) return 0;
    size_t off[5];
    return rescored_parts(t, n, k_cand, off);
}

// csa_index_topk_fp8_rescored and csa_index_topk_fp4_rescored
static int index_topk_lowp_rescored(const void* q, const float* w, const unsigned char* k8, const float* k_scale,
                                    bool fp4, const void* k16, int t, int h_i, int d_i, int n, long long pos0,
                                    int ratio, int top_k, int k_cand, int* idx, int* count, void* ws,
                                    size_t ws_bytes, csa_stream stream, const char* who) {
    CHECK(q && w && idx && ws && ((k8 && k_scale && k16) || n == 0), "%s: null pointer argument", who);
    CHECK(t >= 1 && n >= 0, "%s: t %d n %d", who, t, n);
    CHECK(ratio >= 1, "%s: ratio %d", who, ratio);
    CHECK(top_k >= 1 && k_cand >= top_k && k_cand <= csa::kTopkMaxK,
          "%s: top_k %d / k_cand %d (need 1 <= top_k <= k_cand <= %d)", who, top_k, k_cand, csa::kTopkMaxK);
    if (h_i != 64 || d_i != 128)
        return fail(CSA_ERR_UNSUPPORTED, "%s: needs h_i=64, d_i=128 (got %d, %d)", who, h_i, d_i);
    CHECK(aligned16(q) && aligned16(w) && aligned16(ws) && (n == 0 || (aligned16(k8) && aligned16(k16))),
          "%s: q, w, keys and ws must be 16-byte aligned", who);
    size_t off[5];
    const size_t need = rescored_parts(t, n, k_cand, off);
    if (ws_bytes < need) return fail(CSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", who, ws_bytes, need);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    char* base = static_cast<char*>(ws);
    auto* qc = reinterpret_cast<uint8_t*>(base + off[0]);
    auto* wf = reinterpret_cast<float*>(base + off[1]);
    auto* cand = reinterpret_cast<int*>(base + off[2]);
    auto* ccount = reinterpret_cast<int*>(base + off[3]);
    // 1. the query's codes and folded weights
    hipError_t e = csa::launch_quantize_fp8(q, true, qc, nullptr, static_cast<long long>(t) * 64, 128, s, w, wf);
    if (e != hipSuccess) return launched(e, who);
    // 2. the k_cand best by low-precision score per query
    csa::IndexTopkArgs a{};
    a.w = wf;
    a.t = t;
    a.n = n;
    a.pos0 = pos0;
    a.ratio = ratio;
    a.top_k = k_cand;
    a.idx = cand;
    a.count = ccount;
    a.ws = base + off[4];
    a.q8 = qc;
    a.k8 = k8;
    static const float kNoKeys = 1.f;
    a.k_scale = n > 0 ? k_scale : &kNoKeys;
    a.k_fp4 = fp4 ? 1 : 0;
    e = csa::launch_index_topk(a, s);
    if (e != hipSuccess) return launched(e, who);
    // 3. their exact scores and the top_k of them
    const csa::RescoreRowsArgs r{static_cast<const uint16_t*>(q), w, static_cast<const uint16_t*>(k16), n, cand, ccount,
                                 k_cand, t, top_k, idx, count};
    return launched(csa::launch_rescore_rows(r, s), who);
}

int csa_index_topk_fp8_rescored(const void* q, const float* w, const unsigned char* k8, const float* k_scale,
                                const void* k16, int t, int h_i, int d_i, int n, long long pos0, int ratio, int top_k,
                                int k_cand, int* idx, int* count, void* ws, size_t ws_bytes, csa_stream stream) {
    return index_topk_lowp_rescored(q, w, k8, k_scale, false, k16, t, h_i, d_i, n, pos0, ratio, top_k, k_cand, idx,
                                    count, ws, ws_bytes, stream, "csa_index_topk_fp8_rescored");
}

int csa_index_topk_fp4_rescored(const void* q, const float* w, const unsigned char* k4, const unsigned int* k_scales,
                                const void* k16, int t, int h_i, int d_i, int n, long long pos0, int ratio, int top_k,
                                int k_cand, int* idx, int* count, void* ws, size_t ws_bytes, csa_stream stream) {
    return index_topk_lowp_rescored(q, w, k4, reinterpret_cast<const float*>(k_scales), true, k16, t, h_i, d_i, n,
                                    pos0, ratio, top_k, k_cand, idx, count, ws, ws_bytes, stream,
                                    "csa_index_topk_fp4_rescored");
}

int csa_prefill_attn(const void* q, const void* comp_kv, int n_comp, const int* idx, const int* count, int k,
                     const void* win_kv, int window, long long pos0, const float* sink, float scale, void* out,
                     csa_dtype out_dtype, float* lse, int t, int h, int d, csa_stream stream) {
    CHECK(q && idx && win_kv && out && (comp_kv || n_comp == 0), "csa_prefill_attn: null pointer argument");
    CHECK(t >= 1 && n_comp >= 0, "csa_prefill_attn: t %d n_comp %d", t, n_comp);
    CHECK(k >= 1 && k <= csa::kTopkMaxK, "csa_prefill_attn: k=%d out of 1..%d", k, csa::kTopkMaxK);
    CHECK(window >= 1 && pos0 >= 0, "csa_prefill_attn: window %d / pos0 %lld", window, pos0);
    CHECK(out_dtype == CSA_F32 || out_dtype == CSA_BF16, "csa_prefill_attn: bad out_dtype %d", (int)out_dtype);
    if (!csa::prefill_attn_supported(h, d))
        return fail(CSA_ERR_UNSUPPORTED, "csa_prefill_attn: needs h a multiple of 16 up to 64 and d in {128, 256, 512} "
                    "(got %d, %d)", h, d);
    CHECK(aligned16(q) && aligned16(win_kv) && aligned16(out) && (n_comp == 0 || aligned16(comp_kv)),
          "csa_prefill_attn: q, comp_kv, win_kv and out must be 16-byte aligned");
    csa::PrefillAttnArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(comp_kv), n_comp, idx,
                           count, k, static_cast<const uint16_t*>(win_kv), window, pos0, sink, scale, out,
                           out_dtype == CSA_BF16, lse, t, h, d};
    return launched(csa::launch_prefill_attn(a, static_cast<hipStream_t>(stream)), "csa_prefill_attn");
}

int csa_prefill_attn_mixed(const void* q, const unsigned char* comp_rec, int n_comp, const int* idx, const int* count,
                           int k, const unsigned char* win_rec, int window, long long pos0, const float* rope_cos,
                           const float* rope_sin, int rope_rows, const float* sink, float scale, void* out,
                           csa_dtype out_dtype, float* lse, int t, int h, csa_stream stream) {
    CHECK(q && idx && win_rec && out && (comp_rec || n_comp == 0), "csa_prefill_attn_mixed: null pointer argument");
    CHECK(rope_cos && rope_sin, "csa_prefill_attn_mixed: null RoPE table");
    CHECK(t >= 1 && n_comp >= 0, "csa_prefill_attn_mixed: t %d n_comp %d", t, n_comp);
    CHECK(k >= 1 && k <= csa::kTopkMaxK, "csa_prefill_attn_mixed: k=%d out of 1..%d", k, csa::kTopkMaxK);
    CHECK(window >= 1 && pos0 >= 0, "csa_prefill_attn_mixed: window %d / pos0 %lld", window, pos0);
    CHECK(pos0 + t <= rope_rows, "csa_prefill_attn_mixed: positions up to %lld outside the RoPE table (%d rows)",
          pos0 + t - 1, rope_rows);
    CHECK(out_dtype == CSA_F32 || out_dtype == CSA_BF16, "csa_prefill_attn_mixed: bad out_dtype %d", (int)out_dtype);
    if (!csa::prefill_attn_supported(h, csa::kMixD))
        return fail(CSA_ERR_UNSUPPORTED, "csa_prefill_attn_mixed: needs h a multiple of 16 up to 64 (got %d)", h);
    CHECK(aligned16(q) && aligned16(win_rec) && aligned16(out) && (n_comp == 0 || aligned16(comp_rec)),
          "csa_prefill_attn_mixed: q, comp_rec, win_rec and out must be 16-byte aligned");
    csa::PrefillAttnArgs a{static_cast<const uint16_t*>(q), reinterpret_cast<const uint16_t*>(comp_rec), n_comp, idx,
                           count, k, reinterpret_cast<const uint16_t*>(win_rec), window, pos0, sink, scale, out,
                           out_dtype == CSA_BF16, lse, t, h, csa::kMixD, true, rope_cos, rope_sin};
    return launched(csa::launch_prefill_attn(a, static_cast<hipStream_t>(stream)), "csa_prefill_attn_mixed");
}

}  // extern "C"

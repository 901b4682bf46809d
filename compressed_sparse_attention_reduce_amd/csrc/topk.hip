// Fixed-shape top-k of score rows: the k largest valid scores, ordered by
// score descending then index ascending; unused slots -1 plus a device count.
//
// Page 1, ARCHITECTURE_AND_MEMORY_AUDIT.md, F3 (tk = min(top_k, n_comp),
// total.topk(tk, -1)); page 3, GETTING+CUDAGRAPH_READY.md, Section C item 3
// (fixed k, invalid entries masked, no host read of the count).
//
// Every element gets a unique 64-bit composite  c = key(score) << 32 | ~index
// (key order-preserving, -0 folded onto +0), so "the k largest composites" is
// exactly the wanted set and order whatever the ties.
//
// Cross-workgroup atomics and fences are slow on this chip (hundreds of
// workgroups hitting one address serialise), so the selection uses none:
//   * candidates: every producer workgroup (the score kernel's, or
//     k_topk_cands for a standalone call) writes the top m+1 composites of its
//     own slice to a private slot of the workspace;
//   * k_topk_final, one workgroup per row, loads the union of the kept m per
//     slot into registers and keeps only entries above every slot's bound
//     (entry m + 1 of a slot: at least the largest composite it did not
//     keep).  If k entries remain they are provably the true top k; they are
//     selected and sorted in one go (a radix digit placed where they differ,
//     bin starts giving final positions, ranks inside each bin).
//   * otherwise, in order until one holds the candidates in LDS:
//     - refine (the top k clustered in a few slots, e.g. recent blocks
//       outscoring the cache): the k-th largest listed key bounds the answer
//       from below; the slots whose bound reaches it are re-read from the
//       score row, the others contribute their lists;
//     - two streaming reads of the row (no lists, or many open slots): the
//       k-th largest of the threads' maxima is the bound;
//     - the exact select over the whole row (ties that keep more entries
//       than LDS holds): 12-bit key histogram, threshold bin, further digits
//       until the remaining candidates fit, then the same sorted select.
// Every path is exact; only the time differs.
#include <cmath>

#include "common.h"
#include "kernels.h"
#include "topk_common.h"
#include "topk_final.h"

namespace csa {

namespace {

constexpr int kCandThreads = 256;
constexpr int kCandChunk = 2048;      // scores per k_topk_cands workgroup
constexpr int kCandPer = kCandChunk / kCandThreads;

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

__global__ __launch_bounds__(kFinalThreads) void k_topk_final(TopkArgs a, CandArgs c) {
    if (a.dev) a.n = dev_step_entries(dev_load(a.dev, a.w, a.max_comp), a.m, a.max_comp);
    extern __shared__ __attribute__((aligned(16))) unsigned char final_smem[];
    FinalSmem& sm = *reinterpret_cast<FinalSmem*>(final_smem);
    const int row = blockIdx.x;
    const int b = row / a.t;
    const int tt = row - b * a.t;
    int* out = a.idx + (static_cast<long long>(b) * a.t + tt) * a.k;
    uint32_t k_eff = 0;
    const bool done = c.lists && union_topk(sm, c, row, a.k, out, k_eff);
    if (!done) {
        __syncthreads();  // the fast path's reads of sm are over
        k_eff = row_topk(sm, c, row, score_row(a, row), a.n, a.k, out);
    }
    const int ns = static_cast<int>(k_eff);
    for (int j = ns + threadIdx.x; j < a.k; j += blockDim.x) out[j] = -1;
    if (a.count && threadIdx.x == 0) a.count[static_cast<long long>(b) * a.t + tt] = ns;
}

// Many long rows (the prefill chunk): one workgroup per row selects from the
// row held in registers (long_row_topk), the exact path if that overflows.
__global__ __launch_bounds__(kFinalThreads) void k_topk_long(TopkArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char final_smem[];
    FinalSmem& sm = *reinterpret_cast<FinalSmem*>(final_smem);
    const int row = blockIdx.x;
    const int b = row / a.t;
    const int tt = row - b * a.t;
    int* out = a.idx + (static_cast<long long>(b) * a.t + tt) * a.k;
    uint32_t k_eff = 0;
    if (!long_row_topk(sm, score_row(a, row), a.n, a.k, out, k_eff)) {
        __syncthreads();
        k_eff = exact_row_topk(sm, score_row(a, row), a.n, a.k, out);
    }
    const int ns = static_cast<int>(k_eff);
    for (int j = ns + threadIdx.x; j < a.k; j += blockDim.x) out[j] = -1;
    if (a.count && threadIdx.x == 0) a.count[static_cast<long long>(b) * a.t + tt] = ns;
}

// Standalone candidate producer: each workgroup lists the top m of its chunk
// of scores plus a bound of the rest (the same per-slot lists the score
// kernel writes).
__global__ __launch_bounds__(kCandThreads) void k_topk_cands(TopkArgs a, CandArgs c) {
    __shared__ CandSmem cs;
    const int row = blockIdx.y;
    const float* s = score_row(a, row);
    const long long beg = static_cast<long long>(blockIdx.x) * kCandChunk;
    float x[kCandPer];
#pragma unroll
    for (int u = 0; u < kCandPer; ++u) {
        const long long i = beg + u * kCandThreads + threadIdx.x;
        x[u] = i < a.n ? s[i] : -INFINITY;
    }
    u64 top[kCandPer];
    u64 drop = 0;
#pragma unroll
    for (int u = 0; u < kCandPer; ++u) top[u] = 0;
#pragma unroll
    for (int u = 0; u < kCandPer; ++u) {
        const long long i = beg + u * kCandThreads + threadIdx.x;
        const uint32_t key = score_key(x[u]);
        lane_insert(top, drop, key_valid(key, x[u]) ? composite(key, static_cast<uint32_t>(i)) : 0ull);
    }
    block_top_m<kCandThreads / kWave>(top, drop, c.m, c.mw, c.lists + (static_cast<long long>(row) * c.slots + blockIdx.x) * (c.m + 1), cs);
}

}  // namespace

// k_topk_final takes more than 64 KB of LDS: opt in once per device.
static bool final_lds_opted_in() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    static bool done[64] = {};
    if (!done[dev])
        done[dev] = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_topk_final),
                                        hipFuncAttributeMaxDynamicSharedMemorySize,
                                        static_cast<int>(sizeof(FinalSmem))) == hipSuccess;
    return done[dev];
}

static bool long_lds_opted_in() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    static bool done[64] = {};
    if (!done[dev])
        done[dev] = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_topk_long),
                                        hipFuncAttributeMaxDynamicSharedMemorySize,
                                        static_cast<int>(sizeof(FinalSmem))) == hipSuccess;
    return done[dev];
}

hipError_t launch_topk_rows(const TopkArgs& a, hipStream_t s) {
    const int rows = a.batch * a.t;
    if (rows == 0) return hipSuccess;
    if (a.n > kLongPer * kFinalThreads) return launch_topk(a, nullptr, s);
    if (!long_lds_opted_in()) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_topk_long, dim3(rows), dim3(kFinalThreads), sizeof(FinalSmem), s, a);
    return hipGetLastError();
}

int topk_cand_m(int n, int k, int keys_per_slot) {
    // slots hold m + 1 entries; m covers the expected share e of the top k of
    // a slot plus 4 sqrt(e) + 2 (Poisson tails: about one row in a thousand
    // at 1M context has a slot that held more; the top-k proves containment
    // and then re-reads the few slots concerned)
    if (n <= 0 || keys_per_slot <= 0) return -1;
    const double e = static_cast<double>(k) * keys_per_slot / n;
    const int m = static_cast<int>(e + 4.0 * sqrt(e) + 2.0 + 0.999);
    return m + 1 <= kMaxCandM1 ? m : -1;
}

size_t topk_workspace_bytes(int rows, int n, int k) {
    // per-slot candidate lists of the standalone producer
    const int slots = n > 0 ? (n + kCandChunk - 1) / kCandChunk : 1;
    const int m = topk_cand_m(n, k, kCandChunk);
    return align256(static_cast<size_t>(rows) * slots * (m > 0 ? m + 1 : 1) * sizeof(u64));
}

hipError_t launch_topk(const TopkArgs& a, const CandArgs* cands, hipStream_t s) {
    const int rows = a.batch * a.t;
    if (rows == 0) return hipSuccess;
    CandArgs c{};
    if (cands) {
        c = *cands;
    } else if (a.n > 2 * kCandChunk) {
        // standalone: produce per-chunk candidates when the row is long
        const int slots = (a.n + kCandChunk - 1) / kCandChunk;
        const int m = topk_cand_m(a.n, a.k, kCandChunk);
        const int mw = topk_cand_m(a.n, a.k, kCandChunk / (kCandThreads / kWave));
        if (m > 0) {
            c.lists = static_cast<u64*>(a.ws);
            c.slots = slots;
            c.m = m;
            c.mw = mw < m ? mw : m;
            c.run = kCandChunk;
            c.stride = slots * kCandChunk;
            hipLaunchKernelGGL(k_topk_cands, dim3(slots, rows), dim3(kCandThreads), 0, s, a, c);
        }
    }
    if (!final_lds_opted_in()) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_topk_final, dim3(rows), dim3(kFinalThreads), sizeof(FinalSmem), s, a, c);
    return hipGetLastError();
}

}  // namespace csa

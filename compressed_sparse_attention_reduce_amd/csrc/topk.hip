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
//   * k_topk_final, one workgroup per row, selects the top k of the union of
//     the kept m per slot and checks that every slot's (m+1)-th composite
//     (the largest it dropped) is below the k-th pick, which proves the union
//     held the true top k.  If the check fails (adversarial ties, or no
//     candidates were produced) it runs an exact radix select over the whole
//     row instead: 12-bit key histogram, threshold bin, then further digits of
//     the composite until the remaining candidates fit in LDS.
// Either way the result is exact; only the time differs.
#include <cmath>

#include "common.h"
#include "kernels.h"
#include "topk_common.h"

namespace csa {

namespace {

constexpr int kFinalThreads = 1024;
constexpr int kUnionCap = 8192;       // candidates of the fast path held in LDS
constexpr int kPool = 2048;           // exact-path candidates held in LDS
constexpr int kRefineBits = 10;
constexpr int kCandThreads = 256;
constexpr int kCandChunk = 2048;      // scores per k_topk_cands workgroup

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

__device__ inline const float* score_row(const TopkArgs& a, int row) {
    const int b = row / a.t;
    const int tt = row - b * a.t;
    return a.scores + b * a.s_stride_b + static_cast<long long>(tt) * a.ld_s;
}

// Descending bitonic sort of buf[0..n) in LDS (n a power of two).
__device__ void bitonic_desc(u64* buf, int n) {
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < (n >> 1); i += blockDim.x) {
                const int p = 2 * i - (i & (stride - 1));
                const int q = p + stride;
                const bool desc = (p & size) == 0;
                const u64 x = buf[p], y = buf[q];
                if ((x < y) == desc) { buf[p] = y; buf[q] = x; }
            }
            __syncthreads();
        }
    }
}

__device__ inline int next_pow2(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

// Source of elements for the exact path: the score row (valid entries whose
// key's top 12 bits equal bin12, or all valid entries when bin12 < 0).
__device__ inline bool row_get(const float* row, long long i, int bin12, u64& c) {
    const float x = row[i];
    const uint32_t key = score_key(x);
    if (!key_valid(key, x)) return false;
    if (bin12 >= 0 && static_cast<int>(key >> (32 - kHistBits)) != bin12) return false;
    c = composite(key, static_cast<uint32_t>(i));
    return true;
}

struct FinalSmem {
    u64 sel[kTopkMaxK];        // winners (unordered until the final sort)
    u64 pool[kUnionCap];       // candidates (fast path: the union; exact path: the threshold bin)
    uint32_t hist[kHistBins];
    uint32_t n_sel, n_pool, flag;
    u64 maxdrop;
};

__device__ inline void pool_select(FinalSmem& sm, uint32_t np, uint32_t need, int pb) {
    lds_select(sm.pool, np, need, pb, 1024, pb == 0 ? kHistBits : 8, sm.sel, &sm.n_sel, &sm.n_pool, sm.hist);
}

// Exact top-k of one score row by one workgroup.  Returns k_eff.
__device__ uint32_t exact_row_topk(FinalSmem& sm, const float* row, int n, int k) {
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) sm.hist[i] = 0;
    if (threadIdx.x == 0) { sm.n_sel = 0; sm.n_pool = 0; }
    __syncthreads();
    for (long long i = threadIdx.x; i < n; i += blockDim.x) {
        const float x = row[i];
        const uint32_t key = score_key(x);
        if (key_valid(key, x)) atomicAdd(&sm.hist[key >> (32 - kHistBits)], 1u);
    }
    __syncthreads();
    int tb;
    uint32_t above, at, total;
    block_threshold(sm.hist, kHistBins, static_cast<uint32_t>(k), tb, above, at, total);
    const uint32_t k_eff = tb < 0 ? total : static_cast<uint32_t>(k);
    const bool pool_fits = at <= kPool;
    for (long long base = 0; base < n; base += blockDim.x) {
        const long long i = base + threadIdx.x;
        u64 c = 0;
        int bin = -2;
        if (i < n && row_get(row, i, -1, c)) bin = static_cast<int>(c >> (64 - kHistBits));
        const uint32_t ps = wave_append_pos(bin > tb, &sm.n_sel);
        if (bin > tb) sm.sel[ps] = c;
        const uint32_t pp = wave_append_pos(bin == tb && pool_fits, &sm.n_pool);
        if (bin == tb && pool_fits) sm.pool[pp] = c;
    }
    __syncthreads();
    if (tb < 0) return k_eff;
    uint32_t need = k_eff - above;
    u64 prefix = static_cast<u64>(tb);
    int pb = kHistBits;
    // the threshold bin overflowed the pool: more digits over the row
    while (!pool_fits || sm.n_pool > kPool) {
        const int db = min(kRefineBits, 64 - pb);
        const int nb = 1 << db;
        for (int i = threadIdx.x; i < nb; i += blockDim.x) sm.hist[i] = 0;
        __syncthreads();
        for (long long i = threadIdx.x; i < n; i += blockDim.x) {
            u64 c;
            if (row_get(row, i, tb, c) && (c >> (64 - pb)) == prefix)
                atomicAdd(&sm.hist[(c >> (64 - pb - db)) & (nb - 1)], 1u);
        }
        __syncthreads();
        int td;
        uint32_t ab, at2, tot;
        block_threshold(sm.hist, nb, need, td, ab, at2, tot);
        const bool fits = at2 <= kPool;
        if (threadIdx.x == 0) sm.n_pool = 0;
        __syncthreads();
        for (long long base = 0; base < n; base += blockDim.x) {
            const long long i = base + threadIdx.x;
            u64 c = 0;
            int dg = -2;
            if (i < n && row_get(row, i, tb, c) && (c >> (64 - pb)) == prefix)
                dg = static_cast<int>((c >> (64 - pb - db)) & (nb - 1));
            const uint32_t ps = wave_append_pos(dg > td, &sm.n_sel);
            if (dg > td) sm.sel[ps] = c;
            const uint32_t pp = wave_append_pos(dg == td && fits, &sm.n_pool);
            if (dg == td && fits) sm.pool[pp] = c;
        }
        __syncthreads();
        need -= ab;
        prefix = (prefix << db) | static_cast<u64>(static_cast<uint32_t>(td));
        pb += db;
        if (fits) break;
    }
    pool_select(sm, sm.n_pool, need, pb);
    return k_eff;
}

// Fast path: top-k of the union of per-slot candidates, with the containment
// check.  Returns false if the union cannot prove the answer.
__device__ bool union_topk(FinalSmem& sm, const CandArgs& c, int row, int k) {
    const int slots = c.slots;
    const int m1 = c.m + 1;
    const u64* lists = c.lists + static_cast<long long>(row) * slots * m1;
    if (threadIdx.x == 0) { sm.n_pool = 0; sm.n_sel = 0; sm.maxdrop = 0; sm.flag = 0; }
    __syncthreads();
    // kept entries (first m of every slot) into the pool; the (m+1)-th of each
    // slot is the largest composite that slot dropped.  Loads are batched so
    // their latencies overlap.
    u64 mine = 0;
    const int total = slots * m1;
    constexpr int kBatch = 8;
    for (int base = 0; base < total; base += blockDim.x * kBatch) {
        u64 v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = base + u * blockDim.x + threadIdx.x;
            v[u] = i < total ? lists[i] : 0ull;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = base + u * blockDim.x + threadIdx.x;
            const bool drop = i < total && i % m1 == c.m;
            if (drop) mine = v[u] > mine ? v[u] : mine;
            const bool keep = !drop && v[u] != 0;
            const uint32_t p = wave_append_pos(keep, &sm.n_pool);
            if (keep && p < kUnionCap) sm.pool[p] = v[u];
        }
    }
    // block max of the dropped composites
    for (int o = 32; o > 0; o >>= 1) {
        const u64 other = __shfl_xor(mine, o);
        mine = other > mine ? other : mine;
    }
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) atomicMax(&sm.maxdrop, mine);
    __syncthreads();
    const uint32_t np = sm.n_pool;
    if (np > kUnionCap) return false;
    const u64 maxdrop = sm.maxdrop;
    if (np < static_cast<uint32_t>(k)) {
        // fewer valid candidates than k: exact only if no slot dropped anything valid
        if (maxdrop != 0) return false;
        for (uint32_t i = threadIdx.x; i < np; i += blockDim.x) sm.sel[i] = sm.pool[i];
        __syncthreads();
        if (threadIdx.x == 0) sm.n_sel = np;
        __syncthreads();
        return true;
    }
    pool_select(sm, np, static_cast<uint32_t>(k), 0);
    // containment: the k-th pick must beat everything any slot dropped
    u64 kmin = ~0ull;
    for (int i = threadIdx.x; i < k; i += blockDim.x) kmin = sm.sel[i] < kmin ? sm.sel[i] : kmin;
    for (int o = 32; o > 0; o >>= 1) {
        const u64 other = __shfl_xor(kmin, o);
        kmin = other < kmin ? other : kmin;
    }
    if ((threadIdx.x & (kWave - 1)) == 0 && kmin <= maxdrop) atomicOr(&sm.flag, 1u);
    __syncthreads();
    return sm.flag == 0;
}

__global__ __launch_bounds__(kFinalThreads) void k_topk_final(TopkArgs a, CandArgs c) {
    __shared__ FinalSmem sm;
    const int row = blockIdx.x;
    bool done = false;
    uint32_t k_eff = 0;
    if (c.lists) {
        done = union_topk(sm, c, row, a.k);
        if (done) k_eff = sm.n_sel;
    }
    if (!done) k_eff = exact_row_topk(sm, score_row(a, row), a.n, a.k);
    // final order of the k_eff winners
    const int ns = static_cast<int>(k_eff);
    const int p2 = next_pow2(ns > 1 ? ns : 1);
    for (int i = ns + threadIdx.x; i < p2; i += blockDim.x) sm.sel[i] = 0;
    __syncthreads();
    bitonic_desc(sm.sel, p2);
    const int b = row / a.t;
    const int tt = row - b * a.t;
    int* out = a.idx + (static_cast<long long>(b) * a.t + tt) * a.k;
    for (int j = threadIdx.x; j < a.k; j += blockDim.x) out[j] = j < ns ? composite_index(sm.sel[j]) : -1;
    if (a.count && threadIdx.x == 0) a.count[static_cast<long long>(b) * a.t + tt] = ns;
}

// Standalone candidate producer: each workgroup keeps the top m+1 of its
// chunk of scores (the same per-slot lists the score kernel writes).
__global__ __launch_bounds__(kCandThreads) void k_topk_cands(TopkArgs a, CandArgs c) {
    __shared__ u64 vals[kCandChunk];
    __shared__ CandSmem cs;
    const int row = blockIdx.y;
    const float* s = score_row(a, row);
    const long long beg = static_cast<long long>(blockIdx.x) * kCandChunk;
    constexpr int kPer = kCandChunk / kCandThreads;
    float x[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const long long i = beg + u * kCandThreads + threadIdx.x;
        x[u] = i < a.n ? s[i] : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const long long i = beg + u * kCandThreads + threadIdx.x;
        const uint32_t key = score_key(x[u]);
        vals[u * kCandThreads + threadIdx.x] = key_valid(key, x[u]) ? composite(key, static_cast<uint32_t>(i)) : 0ull;
    }
    __syncthreads();
    block_top_m1(vals, kCandChunk, c.m + 1, c.lists + (static_cast<long long>(row) * c.slots + blockIdx.x) * (c.m + 1), cs);
}

}  // namespace

int topk_cand_m(int n, int k, int keys_per_slot) {
    // slots hold m + 1 entries; m covers the expected share of the top k of a
    // slot plus six standard deviations (the final kernel proves containment
    // and falls back to the exact path if a slot held more)
    if (n <= 0 || keys_per_slot <= 0) return -1;
    const double e = static_cast<double>(k) * keys_per_slot / n;
    const int m = static_cast<int>(e + 6.0 * sqrt(e) + 4.0 + 0.999);
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
        if (m > 0) {
            c.lists = static_cast<u64*>(a.ws);
            c.slots = slots;
            c.m = m;
            hipLaunchKernelGGL(k_topk_cands, dim3(slots, rows), dim3(kCandThreads), 0, s, a, c);
        }
    }
    hipLaunchKernelGGL(k_topk_final, dim3(rows), dim3(kFinalThreads), 0, s, a, c);
    return hipGetLastError();
}

}  // namespace csa

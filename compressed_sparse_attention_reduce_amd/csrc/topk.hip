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
//     bin starts giving final positions, ranks inside each bin).  Otherwise
//     (adversarial ties, or no candidates were produced) it runs an exact
//     select over the whole row: 12-bit key histogram, threshold bin, further
//     digits until the remaining candidates fit in LDS, then the same sorted
//     select over them.
// Either way the result is exact; only the time differs.
#include <cmath>

#include "common.h"
#include "kernels.h"
#include "topk_common.h"

namespace csa {

namespace {

constexpr int kFinalThreads = 1024;
constexpr int kUnionRegs = 8;         // union entries per thread of the fast path
constexpr int kUnionCap = kUnionRegs * kFinalThreads;
constexpr int kPool = 2048;           // exact path: threshold-bin entries held in LDS
constexpr int kRefineBits = 10;
constexpr int kCandThreads = 256;
constexpr int kCandChunk = 2048;      // scores per k_topk_cands workgroup
constexpr int kCandPer = kCandChunk / kCandThreads;
static_assert(kPool + kTopkMaxK <= kUnionCap, "exact-path candidates fit the pool");

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

__device__ inline const float* score_row(const TopkArgs& a, int row) {
    const int b = row / a.t;
    const int tt = row - b * a.t;
    return a.scores + b * a.s_stride_b + static_cast<long long>(tt) * a.ld_s;
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

// Dynamic LDS of k_topk_final (about 100 KB).
struct FinalSmem {
    u64 pool[kUnionCap];                  // candidates of the sorted select
    u64 stage[kTopkMaxK + kStageCap];     // its staging; the exact path's picks above the threshold before
    union {
        uint32_t hist[kHistBins];         // row histograms of the exact path
        SortSmem ss;                      // counters of the sorted select (used after them)
    };
    u64 wmax[16], wmin[16];
    uint32_t wcnt[16];
    uint32_t n_sel, n_pool;
};

// Block maxima of the threads' a and b, in every thread.
__device__ inline void block_max2(FinalSmem& sm, u64& a, u64& b) {
    const int wv = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    a = wave_max_u64(a);
    b = wave_max_u64(b);
    if ((threadIdx.x & (kWave - 1)) == 0) {
        sm.wmax[wv] = a;
        sm.wmin[wv] = b;
    }
    __syncthreads();
    a = 0;
    b = 0;
    for (int w = 0; w < nw; ++w) {
        a = umax64(a, sm.wmax[w]);
        b = umax64(b, sm.wmin[w]);
    }
}

// Exact top-k of one score row by one workgroup, as sorted indices into out.
// Returns k_eff.
__device__ uint32_t exact_row_topk(FinalSmem& sm, const float* row, int n, int k, int* out) {
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
    const bool pool_fits = at <= kPool;
    // picks above the threshold bin go to stage, the bin's entries to pool
    for (long long base = 0; base < n; base += blockDim.x) {
        const long long i = base + threadIdx.x;
        u64 c = 0;
        int bin = -2;
        if (i < n && row_get(row, i, -1, c)) bin = static_cast<int>(c >> (64 - kHistBits));
        const uint32_t ps = wave_append_pos(bin > tb, &sm.n_sel);
        if (bin > tb) sm.stage[ps] = c;
        const uint32_t pp = wave_append_pos(bin == tb && pool_fits, &sm.n_pool);
        if (bin == tb && pool_fits) sm.pool[pp] = c;
    }
    __syncthreads();
    if (tb >= 0) {
        uint32_t need = static_cast<uint32_t>(k) - above;
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
                if (dg > td) sm.stage[ps] = c;
                const uint32_t pp = wave_append_pos(dg == td && fits, &sm.n_pool);
                if (dg == td && fits) sm.pool[pp] = c;
            }
            __syncthreads();
            need -= ab;
            prefix = (prefix << db) | static_cast<u64>(static_cast<uint32_t>(td));
            pb += db;
            if (fits) break;
        }
    }
    // all candidates (the bin's entries, then the picks above it) into the pool
    const uint32_t nb_pool = tb >= 0 ? sm.n_pool : 0u;
    const uint32_t ns = sm.n_sel;
    for (uint32_t i = threadIdx.x; i < ns; i += blockDim.x) sm.pool[nb_pool + i] = sm.stage[i];
    __syncthreads();
    const uint32_t np = nb_pool + ns;
    // they share the top bits where their largest and smallest agree
    u64 hi = 0, lo_c = 0;
    for (uint32_t i = threadIdx.x; i < np; i += blockDim.x) {
        hi = umax64(hi, sm.pool[i]);
        lo_c = umax64(lo_c, ~sm.pool[i]);
    }
    block_max2(sm, hi, lo_c);
    const int pb = np <= 1 ? 0 : __clzll(static_cast<long long>(hi ^ ~lo_c));
    return select_sorted<kUnionRegs>(sm.pool, np, static_cast<uint32_t>(k), pb, out, sm.stage, sm.ss, &sm.n_pool);
}

// Fast path: top-k of the union of per-slot candidates, as sorted indices
// into out.  Returns false if the union cannot prove the answer.
__device__ bool union_topk(FinalSmem& sm, const CandArgs& c, int row, int k, int* out, uint32_t& k_eff) {
    const int m1 = c.m + 1;
    const int total = c.slots * m1;
    if (total > kUnionCap) return false;
    const u64* lists = c.lists + static_cast<long long>(row) * total;
    // kept entries (first m of every slot) into registers; entry m of each
    // slot bounds what that slot did not keep
    u64 v[kUnionRegs];
#pragma unroll
    for (int u = 0; u < kUnionRegs; ++u) {
        const int i = threadIdx.x + u * kFinalThreads;
        v[u] = i < total ? lists[i] : 0ull;
    }
    u64 maxdrop = 0, mx = 0;
#pragma unroll
    for (int u = 0; u < kUnionRegs; ++u) {
        const int i = threadIdx.x + u * kFinalThreads;
        if (i < total && i % m1 == c.m) {
            maxdrop = umax64(maxdrop, v[u]);
            v[u] = 0;
        }
        mx = umax64(mx, v[u]);
    }
    // (the sorted select's bin counters are cleared under the same barrier)
    for (int i = threadIdx.x; i < (1 << kSelBits); i += kFinalThreads) sm.ss.cnt[i] = 0;
    block_max2(sm, maxdrop, mx);
    // only entries above every slot's bound can be proven (they share the
    // top bits where maxdrop and mx agree); the sorted select takes its first
    // pass over them straight from the registers
#pragma unroll
    for (int u = 0; u < kUnionRegs; ++u) v[u] = v[u] > maxdrop ? v[u] : 0ull;
    if (mx <= maxdrop) {  // nothing provable
        if (maxdrop != 0) return false;
        k_eff = 0;
        return true;
    }
    const FirstPass fp = select_first_pass(v, static_cast<uint32_t>(k), __clzll(static_cast<long long>(mx ^ maxdrop)),
                                           out, sm.stage, sm.ss, sm.pool, &sm.n_pool);
    // fewer than k proven entries: exact only if no slot left anything valid out
    if (fp.total < static_cast<uint32_t>(k) && maxdrop != 0) return false;
    k_eff = fp.done ? fp.written
                    : fp.off + select_sorted<kUnionRegs>(sm.pool, fp.np, fp.need, fp.pb, out + fp.off, sm.stage,
                                                         sm.ss, &sm.n_pool);
    return true;
}

__global__ __launch_bounds__(kFinalThreads) void k_topk_final(TopkArgs a, CandArgs c) {
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
    block_top_m(top, drop, c.m, c.mw, c.lists + (static_cast<long long>(row) * c.slots + blockIdx.x) * (c.m + 1), cs);
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
        const int mw = topk_cand_m(a.n, a.k, kCandChunk / (kCandThreads / kWave));
        if (m > 0) {
            c.lists = static_cast<u64*>(a.ws);
            c.slots = slots;
            c.m = m;
            c.mw = mw < m ? mw : m;
            hipLaunchKernelGGL(k_topk_cands, dim3(slots, rows), dim3(kCandThreads), 0, s, a, c);
        }
    }
    if (!final_lds_opted_in()) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_topk_final, dim3(rows), dim3(kFinalThreads), sizeof(FinalSmem), s, a, c);
    return hipGetLastError();
}

}  // namespace csa

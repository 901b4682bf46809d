// Fixed-shape top-k of score rows: the k largest valid scores, ordered by
// score descending then index ascending; unused slots -1 plus a device count.
//
// Page 1, ARCHITECTURE_AND_MEMORY_AUDIT.md, F3 (tk = min(top_k, n_comp),
// total.topk(tk, -1)); page 3, GETTING+CUDAGRAPH_READY.md, Section C item 3
// (fixed k, invalid entries masked, no host read of the count).
//
// Every element gets a unique 64-bit composite  c = key(score) << 32 | ~index
// (key is order preserving, -0 folded onto +0), so "largest k composites" is
// exactly the wanted set and order, whatever the ties; the result does not
// depend on the order in which parallel workers find candidates.
//
// Pipeline for one row of n scores (radix select, most significant digit first):
//   1. histogram of the top 12 key bits (built by the score kernel when fused,
//      otherwise by k_topk_hist) -> threshold bin tb: fewer than k valid
//      elements lie above tb, at least k at or above it;
//   2. k_topk_filter, many workgroups: elements above tb go to the "sure" list
//      (always < k of them), elements in tb to the candidate list;
//   3. k_topk_final, one workgroup per row: keeps the sure list, picks the
//      remaining best candidates (bitonic sort in LDS when they fit, else
//      further 10-bit radix digits over the 64-bit composite), and sorts the
//      k winners.
#include "common.h"
#include "kernels.h"

namespace csa {

namespace {

typedef unsigned long long u64;

constexpr int kFilterThreads = 256;
constexpr int kFilterChunk = 8192;   // scores per filter workgroup
constexpr int kFinalThreads = 1024;
constexpr int kCandLds = 4096;       // candidates sorted in LDS
constexpr int kGlobalCandCap = 16384;
constexpr int kRefineBits = 10;

struct RowWs {
    uint32_t* hist;  // [kHistBins]
    uint32_t* ctr;   // [0] sure count, [1] candidate count
    u64* sure;       // [k]
    u64* cand;       // [cap]
};

// Workspace: all rows' histograms first (contiguous, so the score kernel can
// fill them with a plain row stride), then counters, sure lists, candidates.
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
__host__ __device__ inline int cand_cap(int n) { return n < kGlobalCandCap ? (n > 0 ? n : 1) : kGlobalCandCap; }
struct WsLayout {
    size_t ctr, sure, cand, total;
};
__host__ __device__ inline WsLayout ws_layout(int rows, int n, int k) {
    WsLayout l;
    const size_t r = static_cast<size_t>(rows);
    l.ctr = align256(r * kHistBins * sizeof(uint32_t));
    l.sure = l.ctr + align256(r * 4 * sizeof(uint32_t));
    l.cand = l.sure + align256(r * static_cast<size_t>(k) * sizeof(u64));
    l.total = l.cand + align256(r * static_cast<size_t>(cand_cap(n)) * sizeof(u64));
    return l;
}
__device__ inline RowWs row_ws(void* ws, int row, int rows, int n, int k) {
    const WsLayout l = ws_layout(rows, n, k);
    char* p = static_cast<char*>(ws);
    RowWs r;
    r.hist = reinterpret_cast<uint32_t*>(p) + static_cast<size_t>(row) * kHistBins;
    r.ctr = reinterpret_cast<uint32_t*>(p + l.ctr) + static_cast<size_t>(row) * 4;
    r.sure = reinterpret_cast<u64*>(p + l.sure) + static_cast<size_t>(row) * k;
    r.cand = reinterpret_cast<u64*>(p + l.cand) + static_cast<size_t>(row) * cand_cap(n);
    return r;
}

__device__ inline u64 composite(uint32_t key, uint32_t idx) {
    return (static_cast<u64>(key) << 32) | static_cast<u64>(0xffffffffu - idx);
}
__device__ inline int composite_index(u64 c) {
    return static_cast<int>(0xffffffffu - static_cast<uint32_t>(c));
}

__device__ inline const float* score_row(const TopkArgs& a, int row) {
    const int b = row / a.t;
    const int tt = row - b * a.t;
    return a.scores + b * a.s_stride_b + static_cast<long long>(tt) * a.ld_s;
}

// Block-wide search over a histogram held in LDS: the largest bin `tb` with
// suffix(tb) >= need (suffix(x) = elements in bins >= x).  above =
// suffix(tb + 1), at = hist[tb].  If the total is below `need`, tb = -1 and
// above = total.  `scratch` holds one uint32 per thread.  All threads return
// the same values.
__device__ void find_threshold(const uint32_t* hist, int nbins, uint32_t need, uint32_t* scratch,
                               int* out3, int& tb, uint32_t& above, uint32_t& at) {
    const int nt = blockDim.x;
    const int per = (nbins + nt - 1) / nt;
    const int lo = threadIdx.x * per;
    const int hi = min(lo + per, nbins);
    uint32_t mine = 0;
    for (int i = lo; i < hi; ++i) mine += hist[i];
    scratch[threadIdx.x] = mine;
    if (threadIdx.x == 0) { out3[0] = -1; out3[1] = 0; out3[2] = 0; }
    __syncthreads();
    // inclusive suffix scan (Hillis-Steele) over the per-thread sums
    for (int off = 1; off < nt; off <<= 1) {
        const uint32_t add = (threadIdx.x + off < nt) ? scratch[threadIdx.x + off] : 0u;
        __syncthreads();
        scratch[threadIdx.x] += add;
        __syncthreads();
    }
    const uint32_t incl = scratch[threadIdx.x];
    const uint32_t excl = incl - mine;
    const uint32_t total = scratch[0];
    if (total < need) {
        if (threadIdx.x == 0) { out3[0] = -1; out3[1] = static_cast<int>(total); out3[2] = 0; }
    } else if (excl < need && incl >= need) {
        uint32_t acc = excl;
        for (int i = hi - 1; i >= lo; --i) {
            if (acc + hist[i] >= need) {
                out3[0] = i;
                out3[1] = static_cast<int>(acc);
                out3[2] = static_cast<int>(hist[i]);
                break;
            }
            acc += hist[i];
        }
    }
    __syncthreads();
    tb = out3[0];
    above = static_cast<uint32_t>(out3[1]);
    at = static_cast<uint32_t>(out3[2]);
    __syncthreads();
}

// Append `val` to list[ctr++] for every lane with pred (one atomic per wave).
__device__ inline void wave_append(bool pred, u64 val, uint32_t* ctr, u64* list, uint32_t cap) {
    const u64 mask = __ballot(pred);
    if (mask == 0) return;
    const int lane = threadIdx.x & (kWave - 1);
    const int leader = __ffsll(static_cast<long long>(mask)) - 1;
    uint32_t base = 0;
    if (lane == leader) base = atomicAdd(ctr, static_cast<uint32_t>(__popcll(mask)));
    base = __shfl(base, leader);
    if (pred) {
        const u64 below = lane ? (mask & (~0ull >> (64 - lane))) : 0ull;
        const uint32_t pos = base + static_cast<uint32_t>(__popcll(below));
        if (pos < cap) list[pos] = val;
    }
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

// ---- kernels -------------------------------------------------------------------

__global__ __launch_bounds__(kFilterThreads) void k_topk_clear(void* ws, int rows, int n, int k) {
    RowWs w = row_ws(ws, blockIdx.x, rows, n, k);
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) w.hist[i] = 0;
    if (threadIdx.x < 4) w.ctr[threadIdx.x] = 0;
}

__global__ __launch_bounds__(kFilterThreads) void k_topk_hist(TopkArgs a) {
    __shared__ uint32_t lh[kHistBins];
    const int row = blockIdx.y;
    const float* s = score_row(a, row);
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) lh[i] = 0;
    __syncthreads();
    const long long beg = static_cast<long long>(blockIdx.x) * kFilterChunk;
    const long long end = min(beg + kFilterChunk, static_cast<long long>(a.n));
    for (long long i = beg + threadIdx.x; i < end; i += blockDim.x) {
        const float x = s[i];
        const uint32_t key = score_key(x);
        if (key_valid(key, x)) atomicAdd(&lh[key >> (32 - kHistBits)], 1u);
    }
    __syncthreads();
    RowWs w = row_ws(a.ws, row, a.batch * a.t, a.n, a.k);
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x)
        if (lh[i]) atomicAdd(&w.hist[i], lh[i]);
}

__global__ __launch_bounds__(kFilterThreads) void k_topk_filter(TopkArgs a) {
    __shared__ uint32_t lh[kHistBins];
    __shared__ uint32_t scratch[kFilterThreads];
    __shared__ int res[3];
    const int row = blockIdx.y;
    RowWs w = row_ws(a.ws, row, a.batch * a.t, a.n, a.k);
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) lh[i] = w.hist[i];
    __syncthreads();
    int tb;
    uint32_t above, at;
    find_threshold(lh, kHistBins, static_cast<uint32_t>(a.k), scratch, res, tb, above, at);
    const float* s = score_row(a, row);
    const uint32_t cap = static_cast<uint32_t>(cand_cap(a.n));
    const long long beg = static_cast<long long>(blockIdx.x) * kFilterChunk;
    const long long end = min(beg + kFilterChunk, static_cast<long long>(a.n));
    for (long long base = beg; base < end; base += blockDim.x) {
        const long long i = base + threadIdx.x;
        bool sure = false, cand = false;
        u64 c = 0;
        if (i < end) {
            const float x = s[i];
            const uint32_t key = score_key(x);
            if (key_valid(key, x)) {
                const int bin = static_cast<int>(key >> (32 - kHistBits));
                sure = bin > tb;
                cand = bin == tb;
                c = composite(key, static_cast<uint32_t>(i));
            }
        }
        wave_append(sure, c, &w.ctr[0], w.sure, static_cast<uint32_t>(a.k));
        wave_append(cand, c, &w.ctr[1], w.cand, cap);
    }
}

// Source of candidates for the refinement: a list of composites, or the
// score row itself restricted to keys whose top 12 bits equal the first
// threshold bin.
struct Source {
    const u64* list;
    const float* row;
    long long len;
    uint32_t bin12;
};

__device__ inline bool source_get(const Source& src, long long i, u64& c) {
    if (src.list) {
        c = src.list[i];
        return true;
    }
    const float x = src.row[i];
    const uint32_t key = score_key(x);
    if (!key_valid(key, x) || (key >> (32 - kHistBits)) != src.bin12) return false;
    c = composite(key, static_cast<uint32_t>(i));
    return true;
}

__global__ __launch_bounds__(kFinalThreads) void k_topk_final(TopkArgs a) {
    __shared__ u64 sel[kTopkMaxK];
    __shared__ u64 pool[kCandLds];  // candidates; doubles as histogram space
    __shared__ uint32_t scratch[kFinalThreads];
    __shared__ int res[3];
    __shared__ uint32_t n_sel, n_pool;
    uint32_t* hist = reinterpret_cast<uint32_t*>(pool);

    const int row = blockIdx.x;
    RowWs w = row_ws(a.ws, row, a.batch * a.t, a.n, a.k);
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) hist[i] = w.hist[i];
    __syncthreads();
    int tb;
    uint32_t above, at;
    find_threshold(hist, kHistBins, static_cast<uint32_t>(a.k), scratch, res, tb, above, at);
    const uint32_t k_eff = tb < 0 ? above : static_cast<uint32_t>(a.k);
    const uint32_t n_sure = min(w.ctr[0], k_eff);
    const uint32_t n_cand = w.ctr[1];
    for (uint32_t i = threadIdx.x; i < n_sure; i += blockDim.x) sel[i] = w.sure[i];
    if (threadIdx.x == 0) { n_sel = n_sure; n_pool = 0; }
    __syncthreads();

    uint32_t need = k_eff - n_sure;  // > 0 only if bin tb holds the rest
    if (need > 0) {
        const uint32_t cap = static_cast<uint32_t>(cand_cap(a.n));
        Source src;
        src.list = nullptr;
        src.row = score_row(a, row);
        src.len = a.n;
        src.bin12 = static_cast<uint32_t>(tb);
        if (n_cand <= cap) { src.list = w.cand; src.len = n_cand; }
        bool done = false;
        if (n_cand <= kCandLds) {
            for (uint32_t i = threadIdx.x; i < n_cand; i += blockDim.x) pool[i] = w.cand[i];
            if (threadIdx.x == 0) n_pool = n_cand;
            __syncthreads();
            done = true;
        }
        // Radix refinement over the 64-bit composite: after the 12-bit key
        // digit, 10-bit digits until the remaining candidates fit in LDS.
        u64 prefix = static_cast<u64>(tb);
        int pb = kHistBits;
        while (!done) {
            const int db = min(kRefineBits, 64 - pb);
            const int nb = 1 << db;
            for (int i = threadIdx.x; i < nb; i += blockDim.x) hist[i] = 0;
            __syncthreads();
            for (long long i = threadIdx.x; i < src.len; i += blockDim.x) {
                u64 c;
                if (source_get(src, i, c) && (c >> (64 - pb)) == prefix)
                    atomicAdd(&hist[(c >> (64 - pb - db)) & (nb - 1)], 1u);
            }
            __syncthreads();
            int td;
            uint32_t ab, at2;
            find_threshold(hist, nb, need, scratch, res, td, ab, at2);
            const bool fits = at2 <= kCandLds;
            __syncthreads();  // hist (aliasing pool) is dead from here on
            for (long long i = threadIdx.x; i < src.len; i += blockDim.x) {
                u64 c;
                if (source_get(src, i, c) && (c >> (64 - pb)) == prefix) {
                    const int dg = static_cast<int>((c >> (64 - pb - db)) & (nb - 1));
                    if (dg > td) sel[atomicAdd(&n_sel, 1u)] = c;
                    else if (dg == td && fits) pool[atomicAdd(&n_pool, 1u)] = c;
                }
            }
            __syncthreads();
            need -= ab;
            prefix = (prefix << db) | static_cast<u64>(td);
            pb += db;
            done = fits;
        }
        // best `need` of the pooled candidates
        const int np = static_cast<int>(n_pool);
        const int p2 = next_pow2(np > 1 ? np : 1);
        for (int i = np + threadIdx.x; i < p2; i += blockDim.x) pool[i] = 0;
        __syncthreads();
        bitonic_desc(pool, p2);
        const uint32_t base = n_sel;
        for (uint32_t i = threadIdx.x; i < need; i += blockDim.x) sel[base + i] = pool[i];
        __syncthreads();
    }

    // final order of the k_eff winners
    const int ns = static_cast<int>(k_eff);
    const int p2 = next_pow2(ns > 1 ? ns : 1);
    for (int i = ns + threadIdx.x; i < p2; i += blockDim.x) sel[i] = 0;
    __syncthreads();
    bitonic_desc(sel, p2);
    const int b = row / a.t;
    const int tt = row - b * a.t;
    int* out = a.idx + (static_cast<long long>(b) * a.t + tt) * a.k;
    for (int j = threadIdx.x; j < a.k; j += blockDim.x)
        out[j] = j < ns ? composite_index(sel[j]) : -1;
    if (a.count && threadIdx.x == 0) a.count[static_cast<long long>(b) * a.t + tt] = ns;
}

}  // namespace

size_t topk_workspace_bytes(int rows, int n, int k) { return ws_layout(rows, n, k).total; }

uint32_t* topk_ws_hist(void* ws) { return static_cast<uint32_t*>(ws); }

hipError_t launch_topk_ws_clear(void* ws, int rows, int n, int k, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(k_topk_clear, dim3(rows), dim3(kFilterThreads), 0, s, ws, rows, n, k);
    return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, bool hist_ready, hipStream_t s) {
    const int rows = a.batch * a.t;
    if (rows == 0) return hipSuccess;
    const int chunks = a.n > 0 ? (a.n + kFilterChunk - 1) / kFilterChunk : 0;
    if (!hist_ready) {
        hipLaunchKernelGGL(k_topk_clear, dim3(rows), dim3(kFilterThreads), 0, s, a.ws, rows, a.n, a.k);
        if (chunks)
            hipLaunchKernelGGL(k_topk_hist, dim3(chunks, rows), dim3(kFilterThreads), 0, s, a);
    }
    if (chunks) hipLaunchKernelGGL(k_topk_filter, dim3(chunks, rows), dim3(kFilterThreads), 0, s, a);
    hipLaunchKernelGGL(k_topk_final, dim3(rows), dim3(kFinalThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace csa

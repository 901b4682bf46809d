// Device helpers of the radix top-k, shared by the score kernel (which keeps
// every workgroup's best candidates) and the top-k kernels.
#pragma once

#include "common.h"
#include "kernels.h"

namespace csa {

typedef unsigned long long u64;

constexpr int kHistBits = 12;               // first radix digit: top 12 bits of the score key
constexpr int kHistBins = 1 << kHistBits;

// Unique sort key of an element: order-preserving score key, then the
// inverted index (so equal scores rank the lower index higher).
__device__ inline u64 composite(uint32_t key, uint32_t idx) {
    return (static_cast<u64>(key) << 32) | static_cast<u64>(0xffffffffu - idx);
}
__device__ inline int composite_index(u64 c) { return static_cast<int>(0xffffffffu - static_cast<uint32_t>(c)); }

// Block-wide search over a histogram in LDS: the largest bin `tb` with
// suffix(tb) >= need (suffix(x) = count in bins >= x); above = suffix(tb+1),
// at = hist[tb], total = suffix(0).  If total < need: tb = -1, above = total.
// Every thread returns the same values.  Uses its own LDS scratch.
__device__ inline void block_threshold(const uint32_t* hist, int nbins, uint32_t need, int& tb,
                                       uint32_t& above, uint32_t& at, uint32_t& total) {
    __shared__ uint32_t scan[1024];
    __shared__ uint32_t res[4];
    const int nt = blockDim.x;
    const int per = (nbins + nt - 1) / nt;
    const int lo = threadIdx.x * per;
    const int hi = min(lo + per, nbins);
    uint32_t mine = 0;
    for (int i = lo; i < hi; ++i) mine += hist[i];
    scan[threadIdx.x] = mine;
    if (threadIdx.x == 0) { res[0] = 0xffffffffu; res[1] = 0; res[2] = 0; }
    __syncthreads();
    for (int off = 1; off < nt; off <<= 1) {  // inclusive suffix scan of the per-thread sums
        const uint32_t add = (threadIdx.x + off < nt) ? scan[threadIdx.x + off] : 0u;
        __syncthreads();
        scan[threadIdx.x] += add;
        __syncthreads();
    }
    const uint32_t incl = scan[threadIdx.x];
    const uint32_t excl = incl - mine;
    const uint32_t tot = scan[0];
    if (tot < need) {
        if (threadIdx.x == 0) { res[0] = 0xffffffffu; res[1] = tot; res[2] = 0; }
    } else if (excl < need && incl >= need) {
        uint32_t acc = excl;
        for (int i = hi - 1; i >= lo; --i) {
            if (acc + hist[i] >= need) {
                res[0] = static_cast<uint32_t>(i);
                res[1] = acc;
                res[2] = hist[i];
                break;
            }
            acc += hist[i];
        }
    }
    __syncthreads();
    tb = static_cast<int>(res[0]);
    above = res[1];
    at = res[2];
    total = tot;
    __syncthreads();
}

// Position of this lane's entry when the lanes with `pred` append to a list
// whose length is *ctr: one LDS atomic per wave instead of one per lane (lanes
// hitting one LDS address serialise).  Every lane of the wave must call it;
// the result is meaningful only where pred holds.
__device__ inline uint32_t wave_append_pos(bool pred, uint32_t* ctr) {
    const u64 mask = __ballot(pred);
    if (mask == 0) return 0;
    const int lane = threadIdx.x & (kWave - 1);
    const int leader = __ffsll(static_cast<long long>(mask)) - 1;
    uint32_t base = 0;
    if (lane == leader) base = atomicAdd(ctr, static_cast<uint32_t>(__popcll(mask)));
    base = __shfl(base, leader);
    const u64 below = lane ? (mask & (~0ull >> (64 - lane))) : 0ull;
    return base + static_cast<uint32_t>(__popcll(below));
}

// Select the `need` largest composites of pool[0..np) (LDS, unique; zero
// entries count as the smallest) and append them, in no particular order, to
// sel[*n_sel ..].  While the pool holds more than rank_max entries it is
// narrowed by radix digits of the composite below bit 64 - pb (first digit
// first_bits wide, then 8): entries above the threshold digit are selected,
// entries on it stay in the pool (compacted in place); the rest are picked by
// rank counting.  np >= need.  hist: 1 << max(first_bits, 8) uint32 of LDS.
// Every thread of the block must call it.
__device__ inline void lds_select(u64* pool, uint32_t np, uint32_t need, int pb, uint32_t rank_max, int first_bits,
                                  u64* sel, uint32_t* n_sel, uint32_t* n_pool, uint32_t* hist) {
    int dbits = first_bits;
    while (np > rank_max && pb < 64) {
        const int db = min(dbits, 64 - pb);
        dbits = 8;
        const int nb = 1 << db;
        for (int i = threadIdx.x; i < nb; i += blockDim.x) hist[i] = 0;
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < np; i += blockDim.x)
            atomicAdd(&hist[(pool[i] >> (64 - pb - db)) & (nb - 1)], 1u);
        __syncthreads();
        int td;
        uint32_t ab, at, tot;
        block_threshold(hist, nb, need, td, ab, at, tot);
        if (threadIdx.x == 0) *n_pool = 0;
        __syncthreads();
        for (uint32_t base = 0; base < np; base += blockDim.x) {
            const uint32_t i = base + threadIdx.x;
            u64 c = 0;
            int dg = -1;
            if (i < np) {
                c = pool[i];
                dg = static_cast<int>((c >> (64 - pb - db)) & (nb - 1));
            }
            __syncthreads();  // this block of the pool is read before compaction writes land in it
            const uint32_t ps = wave_append_pos(dg > td, n_sel);
            if (dg > td) sel[ps] = c;
            const uint32_t pp = wave_append_pos(dg == td, n_pool);
            if (dg == td) pool[pp] = c;
            __syncthreads();
        }
        np = *n_pool;
        need -= ab;
        pb += db;
        __syncthreads();
    }
    const uint32_t base = *n_sel;
    // equal (zero) entries share a rank and leave later slots unwritten: those are zero
    for (uint32_t i = threadIdx.x; i < need; i += blockDim.x) sel[base + i] = 0ull;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < np; i += blockDim.x) {
        const u64 c = pool[i];
        uint32_t rank = 0;
        for (uint32_t j = 0; j < np; ++j) rank += pool[j] > c ? 1u : 0u;
        if (rank < need && c != 0) sel[base + rank] = c;
    }
    __syncthreads();
    if (threadIdx.x == 0) *n_sel = base + need;
    __syncthreads();
}

// LDS scratch of block_top_m1.
struct CandSmem {
    uint32_t hist[kHistBins];
    uint32_t n_sel, n_pool;
    u64 sel[kMaxCandM1];
};

// The m1 largest composites of vals[0..nv) (LDS; zero entries are empty),
// written sorted descending to out[0..m1), zero padded (nv >= m1; vals is
// reordered).  Every thread of the block must call it.
__device__ inline void block_top_m1(u64* vals, int nv, int m1, u64* out, CandSmem& cs) {
    if (threadIdx.x == 0) { cs.n_sel = 0; cs.n_pool = 0; }
    __syncthreads();
    lds_select(vals, static_cast<uint32_t>(nv), static_cast<uint32_t>(m1), 0, 128, kHistBits, cs.sel, &cs.n_sel,
               &cs.n_pool, cs.hist);
    // sort the picks by rank (at most kMaxCandM1 of them; empty picks are 0)
    for (int i = threadIdx.x; i < m1; i += blockDim.x) {
        const u64 c = cs.sel[i];
        uint32_t rank = 0;
        for (int j = 0; j < m1; ++j) rank += (cs.sel[j] > c || (cs.sel[j] == c && j < i)) ? 1u : 0u;
        out[rank] = c;
    }
    __syncthreads();
}

}  // namespace csa

// The exact top-k of one score row by one 1024-thread workgroup, shared by
// the top-k kernel (topk.hip) and the fused top-k + attention kernel of the
// decode step (step_attn.hip).  See topk.hip for the method and its sources.
#pragma once

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
static_assert(kPool + kTopkMaxK <= kUnionCap, "exact-path candidates fit the pool");

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
    uint32_t wcnt[16], wcnt2[16];
    uint32_t n_sel, n_pool;
};

// Block maxima of the threads' a and b, in every thread: lane reductions,
// one LDS exchange of the wave results (one read per lane), lane reductions.
__device__ inline void block_max2(FinalSmem& sm, u64& a, u64& b) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    a = wave_max_u64(a);
    b = wave_max_u64(b);
    if (lane == 0) {
        sm.wmax[wv] = a;
        sm.wmin[wv] = b;
    }
    __syncthreads();
    a = wave_max_u64(lane < nw ? sm.wmax[lane] : 0ull);
    b = wave_max_u64(lane < nw ? sm.wmin[lane] : 0ull);
}

// The same for 32-bit values.
__device__ inline void block_max2_u32(FinalSmem& sm, uint32_t& a, uint32_t& b) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    a = wave_max_u32(a);
    b = wave_max_u32(b);
    if (lane == 0) {
        sm.wcnt[wv] = a;
        sm.wcnt2[wv] = b;
    }
    __syncthreads();
    a = wave_max_u32(lane < nw ? sm.wcnt[lane] : 0u);
    b = wave_max_u32(lane < nw ? sm.wcnt2[lane] : 0u);
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

// Long rows (n <= kLongPer * blockDim.x): the k-th largest of the threads'
// maxima bounds the k-th largest score from below (at least k entries, the
// maxima themselves, are not smaller), so every entry in or above the
// histogram bin of that maximum is a candidate and the top k are among them.
// For independent scores that is about 1.5 k - 4 k entries out of n; a second
// read of the row (from L2) compacts them into the pool for the sorted
// select.  Returns false (nothing written) when the candidates overflow the
// pool — heavily tied scores — and the caller takes the exact path.
constexpr int kLongPer = 64;
__device__ inline uint32_t long_key(const float* row, int i, int n) {
    const float x = i < n ? row[i] : -INFINITY;
    const uint32_t kk = score_key(x);
    return key_valid(kk, x) ? kk : 0u;
}
__device__ bool long_row_topk(FinalSmem& sm, const float* row, int n, int k, int* out, uint32_t& k_eff) {
    if (n > kLongPer * static_cast<int>(blockDim.x)) return false;
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t tmax = 0;
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {  // a batch of kLongPer / 2 loads in flight
        uint32_t key[kLongPer / 2];
#pragma unroll
        for (int u = 0; u < kLongPer / 2; ++u) key[u] = long_key(row, (h * kLongPer / 2 + u) * blockDim.x + threadIdx.x, n);
#pragma unroll
        for (int u = 0; u < kLongPer / 2; ++u) tmax = key[u] > tmax ? key[u] : tmax;
    }
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) sm.hist[i] = 0;
    if (threadIdx.x == 0) { sm.n_sel = 0; sm.n_pool = 0; }
    __syncthreads();
    if (tmax) atomicAdd(&sm.hist[tmax >> (32 - kHistBits)], 1u);
    __syncthreads();
    int tb;
    uint32_t above, at, total;
    block_threshold(sm.hist, kHistBins, static_cast<uint32_t>(k), tb, above, at, total);
    // fewer than k thread maxima: every valid entry is a candidate (invalid
    // entries hold key 0, below every valid key)
    const uint32_t edge = tb >= 0 ? static_cast<uint32_t>(tb) << (32 - kHistBits) : 0u;
    const uint32_t lo = edge > kKeyNegInf ? edge : kKeyNegInf + 1;
    // second read: each half's candidates go straight to the pool; every wave
    // reserves its slots with one counter bump (a scan over its lanes)
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
        uint32_t key[kLongPer / 2];
#pragma unroll
        for (int u = 0; u < kLongPer / 2; ++u) key[u] = long_key(row, (h * kLongPer / 2 + u) * blockDim.x + threadIdx.x, n);
        uint32_t c = 0;
#pragma unroll
        for (int u = 0; u < kLongPer / 2; ++u) c += key[u] >= lo ? 1u : 0u;
        uint32_t pre = c, sum = c;
#define CSA_SCAN_STEP(o)                              \
        {                                             \
            const uint32_t other = xor_lanes<o>(sum); \
            if (lane & (o)) pre += other;             \
            sum += other;                             \
        }
        CSA_SCAN_STEP(1) CSA_SCAN_STEP(2) CSA_SCAN_STEP(4) CSA_SCAN_STEP(8) CSA_SCAN_STEP(16) CSA_SCAN_STEP(32)
#undef CSA_SCAN_STEP
        uint32_t base = 0;
        if (lane == 0 && sum) base = atomicAdd(&sm.n_sel, sum);
        base = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(base)));
        uint32_t off = base + pre - c;
        if (base + sum <= static_cast<uint32_t>(kUnionCap)) {  // else overflow: the total shows it
#pragma unroll
            for (int u = 0; u < kLongPer / 2; ++u)
                if (key[u] >= lo)
                    sm.pool[off++] = composite(key[u], static_cast<uint32_t>((h * kLongPer / 2 + u) * blockDim.x +
                                                                             threadIdx.x));
        }
    }
    __syncthreads();
    const uint32_t np = sm.n_sel;
    if (np > static_cast<uint32_t>(kUnionCap)) return false;
    // they share the top bits where their largest and smallest agree
    u64 hi = 0, lo_c = 0;
    for (uint32_t i = threadIdx.x; i < np; i += blockDim.x) {
        hi = umax64(hi, sm.pool[i]);
        lo_c = umax64(lo_c, ~sm.pool[i]);
    }
    block_max2(sm, hi, lo_c);
    const int pb = np <= 1 ? 0 : __clzll(static_cast<long long>(hi ^ ~lo_c));
    k_eff = select_sorted<kUnionRegs>(sm.pool, np, static_cast<uint32_t>(k), pb, out, sm.stage, sm.ss, &sm.n_pool);
    return true;
}

// Rows of any length, in two streaming reads (long_row_topk's bound without
// holding the row): thread t first takes the maximum of its elements t,
// t + blockDim, ...; the k-th largest of those maxima bounds the k-th largest
// score from below, so every entry in or above its 12-bit histogram bin is a
// candidate; the second read compacts them into the pool for the sorted
// select.  Strided elements spread a run of high scores over every thread, so
// scores clustered by index (recent blocks) keep the candidates few.
// Returns false (nothing written) when they overflow the pool (heavily tied
// scores); the caller then takes the exact path.
constexpr int kStreamBatch = 16;  // loads in flight per thread
__device__ bool stream_row_topk(FinalSmem& sm, const float* row, int n, int k, int* out, uint32_t& k_eff) {
    const int lane = threadIdx.x & (kWave - 1);
    const int step = kStreamBatch * static_cast<int>(blockDim.x);
    uint32_t tmax = 0;
#pragma unroll 1
    for (int base = 0; base < n; base += step) {
        uint32_t key[kStreamBatch];
#pragma unroll
        for (int u = 0; u < kStreamBatch; ++u) key[u] = long_key(row, base + u * static_cast<int>(blockDim.x) + threadIdx.x, n);
#pragma unroll
        for (int u = 0; u < kStreamBatch; ++u) tmax = key[u] > tmax ? key[u] : tmax;
    }
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) sm.hist[i] = 0;
    if (threadIdx.x == 0) { sm.n_sel = 0; sm.n_pool = 0; }
    __syncthreads();
    if (tmax) atomicAdd(&sm.hist[tmax >> (32 - kHistBits)], 1u);
    __syncthreads();
    int tb;
    uint32_t above, at, total;
    block_threshold(sm.hist, kHistBins, static_cast<uint32_t>(k), tb, above, at, total);
    // fewer than k thread maxima: every valid entry is a candidate
    const uint32_t edge = tb >= 0 ? static_cast<uint32_t>(tb) << (32 - kHistBits) : 0u;
    const uint32_t lo = edge > kKeyNegInf ? edge : kKeyNegInf + 1;
#pragma unroll 1
    for (int base = 0; base < n; base += step) {
        uint32_t key[kStreamBatch];
#pragma unroll
        for (int u = 0; u < kStreamBatch; ++u) key[u] = long_key(row, base + u * static_cast<int>(blockDim.x) + threadIdx.x, n);
        uint32_t c = 0;
#pragma unroll
        for (int u = 0; u < kStreamBatch; ++u) c += key[u] >= lo ? 1u : 0u;
        uint32_t pre = c, sum = c;
#define CSA_SCAN_STEP(o)                              \
        {                                             \
            const uint32_t other = xor_lanes<o>(sum); \
            if (lane & (o)) pre += other;             \
            sum += other;                             \
        }
        CSA_SCAN_STEP(1) CSA_SCAN_STEP(2) CSA_SCAN_STEP(4) CSA_SCAN_STEP(8) CSA_SCAN_STEP(16) CSA_SCAN_STEP(32)
#undef CSA_SCAN_STEP
        uint32_t wbase = 0;
        if (lane == 0 && sum) wbase = atomicAdd(&sm.n_sel, sum);
        wbase = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(wbase)));
        uint32_t off = wbase + pre - c;
        if (wbase + sum <= static_cast<uint32_t>(kUnionCap)) {  // else overflow: the total shows it
#pragma unroll
            for (int u = 0; u < kStreamBatch; ++u)
                if (key[u] >= lo)
                    sm.pool[off++] = composite(key[u], static_cast<uint32_t>(base + u * static_cast<int>(blockDim.x) +
                                                                            threadIdx.x));
        }
    }
    __syncthreads();
    const uint32_t np = sm.n_sel;
    if (np > static_cast<uint32_t>(kUnionCap)) return false;
    u64 hi = 0, lo_c = 0;
    for (uint32_t i = threadIdx.x; i < np; i += blockDim.x) {
        hi = umax64(hi, sm.pool[i]);
        lo_c = umax64(lo_c, ~sm.pool[i]);
    }
    block_max2(sm, hi, lo_c);
    const int pb = np <= 1 ? 0 : __clzll(static_cast<long long>(hi ^ ~lo_c));
    k_eff = select_sorted<kUnionRegs>(sm.pool, np, static_cast<uint32_t>(k), pb, out, sm.stage, sm.ss, &sm.n_pool);
    return true;
}

// The candidate lists when they cannot prove the top k by themselves: the
// k-th largest listed composite still bounds the k-th largest score from
// below, so the top k lies among the listed entries at or above a lower bound
// of it (two 12-bit digits of the key) and among the unlisted entries of the
// slots whose bound reaches it ("open" slots).  The open slots' keys (as
// c.run / c.stride lay them out) are read again from the score row; the
// other slots contribute their lists, except entries whose key an open slot
// covers (the new key's slot), so no index enters twice.  When the recent
// keys outscore the rest of the cache, only the slots that hold them open and
// a small part of the row is read.  Returns false (nothing written) when the
// layout is not stated, the open slots cover more than a quarter of the row,
// or the candidates overflow the pool.
constexpr int kRefineMaxSlots = 2048;
constexpr int kRefineMaxRuns = 2048;  // (open slot, run) pairs re-read
static_assert(sizeof(FinalSmem::stage) >= (kRefineMaxSlots + kRefineMaxRuns) * sizeof(uint32_t),
              "open-slot list and run starts fit the stage");
__device__ bool refine_topk(FinalSmem& sm, const CandArgs& c, int row, const float* srow, int n, int k, int* out,
                            uint32_t& k_eff) {
    if (!c.lists || c.run <= 0 || (c.run & (c.run - 1)) != 0 || c.stride < c.run || c.stride % c.run != 0 ||
        c.stride / c.run > c.slots || c.slots > kRefineMaxSlots)
        return false;
    const int m1 = c.m + 1;
    const int total = c.slots * m1;
    if (total > kUnionCap) return false;
    const u64* lists = c.lists + static_cast<long long>(row) * total;
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t* hist = sm.hist;
    uint32_t* open_list = reinterpret_cast<uint32_t*>(sm.stage);
    u64 v[kUnionRegs];
#pragma unroll
    for (int u = 0; u < kUnionRegs; ++u) {
        const int i = threadIdx.x + u * kFinalThreads;
        v[u] = i < total ? lists[i] : 0ull;
    }
    // entry i = t + 1024 u is entry i % m1 of slot i / m1 (slot m1 entries: m listed, then the bound);
    // the quotient and remainder advance by fixed steps (one division per thread)
    int sl[kUnionRegs];
    bool bnd[kUnionRegs];
    {
        int q = static_cast<int>(threadIdx.x) / m1;
        int r = static_cast<int>(threadIdx.x) - q * m1;
        const int dq = kFinalThreads / m1, dr = kFinalThreads - dq * m1;
#pragma unroll
        for (int u = 0; u < kUnionRegs; ++u) {
            const bool in = static_cast<int>(threadIdx.x) + u * kFinalThreads < total;
            sl[u] = in ? q : -1;
            bnd[u] = in && r == c.m;
            q += dq;
            r += dr;
            if (r >= m1) {
                r -= m1;
                ++q;
            }
        }
    }
    // 1. a lower bound of the k-th largest listed key: its top 12 bits, then the next 12
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) hist[i] = 0;
    if (threadIdx.x == 0) { sm.n_sel = 0; sm.n_pool = 0; }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kUnionRegs; ++u) {
        const uint32_t hi = static_cast<uint32_t>(v[u] >> 32);
        if (!bnd[u] && hi) atomicAdd(&hist[hi >> 20], 1u);
    }
    __syncthreads();
    int tb;
    uint32_t above, at, listed;
    block_threshold(hist, kHistBins, static_cast<uint32_t>(k), tb, above, at, listed);
    uint32_t edge = 0;
    if (tb >= 0) {
        for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kUnionRegs; ++u) {
            const uint32_t hi = static_cast<uint32_t>(v[u] >> 32);
            if (!bnd[u] && hi && static_cast<int>(hi >> 20) == tb) atomicAdd(&hist[(hi >> 8) & 0xfffu], 1u);
        }
        __syncthreads();
        int tb2;
        uint32_t a2, t2, n2;
        block_threshold(hist, kHistBins, static_cast<uint32_t>(k) - above, tb2, a2, t2, n2);
        edge = (static_cast<uint32_t>(tb) << 20) | (static_cast<uint32_t>(tb2 < 0 ? 0 : tb2) << 8);
    }
    const uint32_t lo = edge > kKeyNegInf ? edge : kKeyNegInf + 1;
    // 2. open slots: flags in hist (one word per slot), their indices in the stage
    for (int i = threadIdx.x; i < c.slots; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    const int layout_slots = c.stride / c.run;  // slots past these list their keys in full
    int unmapped = 0;                            // an open slot outside the layout
#pragma unroll
    for (int u = 0; u < kUnionRegs; ++u) {
        const bool reach = bnd[u] && static_cast<uint32_t>(v[u] >> 32) >= lo;
        const bool open = reach && sl[u] < layout_slots;
        unmapped |= reach && !open;
        const uint32_t p = wave_append_pos(open, &sm.n_pool);
        if (open) {
            hist[sl[u]] = 1u;
            open_list[p] = static_cast<uint32_t>(sl[u]);
        }
    }
    if (__syncthreads_or(unmapped)) return false;
    const uint32_t n_open = sm.n_pool;
    const uint32_t runs = static_cast<uint32_t>((static_cast<long long>(n) + c.stride - 1) / c.stride);
    const long long n_runs_ll = static_cast<long long>(n_open) * runs;
    const long long span_ll = n_runs_ll * c.run;
    if (span_ll > n / 4 + c.run || n_runs_ll > kRefineMaxRuns) return false;  // the streaming reads are cheaper
    const uint32_t n_runs = static_cast<uint32_t>(n_runs_ll);
    const uint32_t span = static_cast<uint32_t>(span_ll);
    // the first key of every (open slot, run) pair: run q is run q % runs of open slot q / runs
    uint32_t* run_start = open_list + kRefineMaxSlots;
    const uint32_t run = static_cast<uint32_t>(c.run), stride = static_cast<uint32_t>(c.stride);
    for (uint32_t q = threadIdx.x; q < n_runs; q += blockDim.x) {
        const uint32_t o = q / runs;
        run_start[q] = open_list[o] * run + (q - o * runs) * stride;
    }
    // 3. candidates: listed entries at or above lo whose key no open slot covers ...
    {
        bool keep[kUnionRegs];
        uint32_t cnt = 0;
#pragma unroll
        for (int u = 0; u < kUnionRegs; ++u) {
            const uint32_t hi = static_cast<uint32_t>(v[u] >> 32);
            keep[u] = sl[u] >= 0 && !bnd[u] && hi >= lo;
            if (keep[u]) {
                const uint32_t idx = ~static_cast<uint32_t>(v[u]);
                keep[u] = hist[(idx % static_cast<uint32_t>(c.stride)) / static_cast<uint32_t>(c.run)] == 0u;
            }
            cnt += keep[u] ? 1u : 0u;
        }
        uint32_t pre = cnt, sum = cnt;
#define CSA_SCAN_STEP(o)                              \
        {                                             \
            const uint32_t other = xor_lanes<o>(sum); \
            if (lane & (o)) pre += other;             \
            sum += other;                             \
        }
        CSA_SCAN_STEP(1) CSA_SCAN_STEP(2) CSA_SCAN_STEP(4) CSA_SCAN_STEP(8) CSA_SCAN_STEP(16) CSA_SCAN_STEP(32)
#undef CSA_SCAN_STEP
        uint32_t wbase = 0;
        if (lane == 0 && sum) wbase = atomicAdd(&sm.n_sel, sum);
        wbase = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(wbase)));
        uint32_t off = wbase + pre - cnt;
        if (wbase + sum <= static_cast<uint32_t>(kUnionCap)) {
#pragma unroll
            for (int u = 0; u < kUnionRegs; ++u)
                if (keep[u]) sm.pool[off++] = v[u];
        }
    }
    // ... and the open slots' keys at or above lo, read from the score row
    // (the runs are powers of two: key f of the re-read is key f % run of run f / run)
    __syncthreads();
    const int run_shift = __ffs(static_cast<int>(run)) - 1;
#pragma unroll 1
    for (uint32_t base = 0; base < span; base += kStreamBatch * blockDim.x) {
        uint32_t key[kStreamBatch];
        int at_i[kStreamBatch];
#pragma unroll
        for (int u = 0; u < kStreamBatch; ++u) {
            const uint32_t f = base + u * blockDim.x + threadIdx.x;
            const int x = f < span ? static_cast<int>(run_start[f >> run_shift] + (f & (run - 1))) : n;  // past the row: key 0
            at_i[u] = x;
            key[u] = long_key(srow, x, n);
        }
        // one slot reservation per wave and batch (a scan of the lanes' counts)
        uint32_t cnt = 0;
#pragma unroll
        for (int u = 0; u < kStreamBatch; ++u) cnt += key[u] >= lo ? 1u : 0u;
        uint32_t pre = cnt, sum = cnt;
#define CSA_SCAN_STEP(o)                              \
        {                                             \
            const uint32_t other = xor_lanes<o>(sum); \
            if (lane & (o)) pre += other;             \
            sum += other;                             \
        }
        CSA_SCAN_STEP(1) CSA_SCAN_STEP(2) CSA_SCAN_STEP(4) CSA_SCAN_STEP(8) CSA_SCAN_STEP(16) CSA_SCAN_STEP(32)
#undef CSA_SCAN_STEP
        uint32_t wbase = 0;
        if (lane == 0 && sum) wbase = atomicAdd(&sm.n_sel, sum);
        wbase = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(wbase)));
        uint32_t off = wbase + pre - cnt;
        if (wbase + sum <= static_cast<uint32_t>(kUnionCap)) {  // else overflow: the total shows it
#pragma unroll
            for (int u = 0; u < kStreamBatch; ++u)
                if (key[u] >= lo) sm.pool[off++] = composite(key[u], static_cast<uint32_t>(at_i[u]));
        }
    }
    __syncthreads();
    const uint32_t np = sm.n_sel;
    if (np > static_cast<uint32_t>(kUnionCap)) return false;
    // 4. the sorted select over them (it reuses the hist words and the stage)
    u64 hi = 0, lo_c = 0;
    for (uint32_t i = threadIdx.x; i < np; i += blockDim.x) {
        hi = umax64(hi, sm.pool[i]);
        lo_c = umax64(lo_c, ~sm.pool[i]);
    }
    block_max2(sm, hi, lo_c);
    const int pb = np <= 1 ? 0 : __clzll(static_cast<long long>(hi ^ ~lo_c));
    k_eff = select_sorted<kUnionRegs>(sm.pool, np, static_cast<uint32_t>(k), pb, out, sm.stage, sm.ss, &sm.n_pool);
    return true;
}

// The exact top-k of a row once the candidate lists alone cannot prove it:
// the lists refined by a partial re-read, else the two streaming reads of
// stream_row_topk, else the exact radix path when tied scores overflow them.
__device__ inline uint32_t row_topk(FinalSmem& sm, const CandArgs& c, int row, const float* srow, int n, int k,
                                    int* out) {
    uint32_t k_eff = 0;
    if (refine_topk(sm, c, row, srow, n, k, out, k_eff)) return k_eff;
    __syncthreads();
    if (stream_row_topk(sm, srow, n, k, out, k_eff)) return k_eff;
    __syncthreads();  // the streaming path's LDS reads are over
    return exact_row_topk(sm, srow, n, k, out);
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
    // The bound test only needs the score-key words (the high 32 bits): the
    // largest bound rounded up to the end of its key is still an upper bound
    // of everything the slots left out, and entries above it are provable.
    uint32_t drop_hi = 0, mx_hi = 0;
    // entry i is a slot's bound when i % m1 == m; i = t + u * kFinalThreads,
    // so the remainder advances by a fixed step (no division per entry)
    const int rstep = kFinalThreads % m1;
    int rem = static_cast<int>(threadIdx.x) % m1;
#pragma unroll
    for (int u = 0; u < kUnionRegs; ++u) {
        const uint32_t hi = static_cast<uint32_t>(v[u] >> 32);
        if (rem == c.m) {
            drop_hi = hi > drop_hi ? hi : drop_hi;
            v[u] = 0;
        } else {
            mx_hi = hi > mx_hi ? hi : mx_hi;
        }
        rem += rstep;
        rem -= rem >= m1 ? m1 : 0;
    }
    // (the sorted select's bin counters are cleared under the same barrier)
    for (int i = threadIdx.x; i < (1 << kSelBits); i += kFinalThreads) sm.ss.cnt[i] = 0;
    block_max2_u32(sm, drop_hi, mx_hi);
    const u64 maxdrop = drop_hi ? ((static_cast<u64>(drop_hi) << 32) | 0xffffffffull) : 0ull;
    // only entries above every slot's bound can be proven (they share the
    // top bits where the key words of maxdrop and the largest entry agree);
    // the sorted select takes its first pass over them straight from the
    // registers
#pragma unroll
    for (int u = 0; u < kUnionRegs; ++u) v[u] = v[u] > maxdrop ? v[u] : 0ull;
    if (mx_hi <= drop_hi) {  // nothing provable
        if (maxdrop != 0) return false;
        k_eff = 0;
        return true;
    }
    const int pb = __clz(static_cast<int>(mx_hi ^ drop_hi));
    const FirstPass fp = select_first_pass(v, static_cast<uint32_t>(k), pb, out, sm.stage, sm.ss, sm.pool,
                                           &sm.n_pool);
    // fewer than k proven entries: exact only if no slot left anything valid out
    if (fp.total < static_cast<uint32_t>(k) && maxdrop != 0) return false;
    k_eff = fp.done ? fp.written
                    : fp.off + select_sorted<kUnionRegs>(sm.pool, fp.np, fp.need, fp.pb, out + fp.off, sm.stage,
                                                         sm.ss, &sm.n_pool);
    return true;
}

}  // namespace

}  // namespace csa

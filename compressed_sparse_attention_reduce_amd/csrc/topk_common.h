// Device helpers of the top-k, shared by the score kernel (which keeps every
// workgroup's best candidates) and the top-k kernels.
//
// Everything here works on unique 64-bit composites (order-preserving score
// key << 32 | inverted index; zero means "no element"), so a set of the n
// largest is unique and ties need no special handling.  The helpers are built
// to keep barriers and LDS round trips few: per-lane sorted lists, wave-wide
// exchanges through DPP and permlane swaps, register-resident candidate pools.
#pragma once

#include "common.h"
#include "kernels.h"

namespace csa {

typedef unsigned long long u64;

constexpr int kHistBits = 12;               // first radix digit over a raw score row
constexpr int kHistBins = 1 << kHistBits;
constexpr int kSelBits = 10;                // digits of the register-resident sorted select

// Unique sort key of an element: order-preserving score key, then the
// inverted index (so equal scores rank the lower index higher).
__device__ inline u64 composite(uint32_t key, uint32_t idx) {
    return (static_cast<u64>(key) << 32) | static_cast<u64>(0xffffffffu - idx);
}
__device__ inline int composite_index(u64 c) { return static_cast<int>(0xffffffffu - static_cast<uint32_t>(c)); }

__device__ inline u64 umax64(u64 a, u64 b) { return a > b ? a : b; }
__device__ inline u64 umin64(u64 a, u64 b) { return a < b ? a : b; }

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
    base = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(base), leader));
    const u64 below = lane ? (mask & (~0ull >> (64 - lane))) : 0ull;
    return base + static_cast<uint32_t>(__popcll(below));
}

// Block-wide search over a histogram in LDS: the largest bin tb with
// suffix(tb) >= need, where suffix(x) counts the entries in bins >= x;
// above = suffix(tb + 1), at = hist[tb], total = suffix(0).  If total < need:
// tb = -1 and above = total.  Thread t owns a run of bins counted from the
// top, so the suffix sums are prefix sums over threads: a butterfly inside
// each wave, one LDS exchange of the wave totals.  Every thread returns the
// same values.  At most 16 waves.
__device__ inline void block_threshold(const uint32_t* hist, int nbins, uint32_t need, int& tb,
                                       uint32_t& above, uint32_t& at, uint32_t& total) {
    __shared__ uint32_t wsum[16];
    __shared__ uint32_t res[3];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    const int per = (nbins + blockDim.x - 1) / blockDim.x;
    const int hi = max(nbins - per * static_cast<int>(threadIdx.x), 0);  // bins [lo, hi)
    const int lo = max(hi - per, 0);
    uint32_t mine = 0;
    for (int b = lo; b < hi; ++b) mine += hist[b];
    // inclusive prefix over the lanes: blocks of 2o lanes merge, the upper half adding the lower's total
    uint32_t pre = mine, sum = mine;
#define CSA_SCAN_STEP(o)                                         \
    {                                                            \
        const uint32_t other = xor_lanes<o>(sum);                \
        if (lane & (o)) pre += other;                            \
        sum += other;                                            \
    }
    CSA_SCAN_STEP(1) CSA_SCAN_STEP(2) CSA_SCAN_STEP(4) CSA_SCAN_STEP(8) CSA_SCAN_STEP(16) CSA_SCAN_STEP(32)
#undef CSA_SCAN_STEP
    if (lane == 0) wsum[wv] = sum;
    if (threadIdx.x == 0) { res[0] = 0xffffffffu; res[1] = 0; res[2] = 0; }
    __syncthreads();
    const uint32_t wt = lane < nw ? wsum[lane] : 0u;
    const uint32_t tot = wave_sum_u32(wt);
    const uint32_t before = wave_sum_u32(lane < wv ? wt : 0u);
    const uint32_t incl = before + pre;  // entries in bins >= lo
    const uint32_t excl = incl - mine;   // entries in bins >= hi
    if (tot < need) {
        if (threadIdx.x == 0) res[1] = tot;
    } else if (excl < need && incl >= need) {
        uint32_t acc = excl;
        for (int b = hi - 1; b >= lo; --b) {
            if (acc + hist[b] >= need) {
                res[0] = static_cast<uint32_t>(b);
                res[1] = acc;
                res[2] = hist[b];
                break;
            }
            acc += hist[b];
        }
    }
    __syncthreads();
    tb = static_cast<int>(res[0]);
    above = res[1];
    at = res[2];
    total = tot;
    __syncthreads();
}

// ---- per-lane lists and the workgroup candidate list --------------------------------

// Insert c into a lane's descending list; whatever falls off the end raises
// `drop` (the largest composite this lane discarded).
template <int L>
__device__ inline void lane_insert(u64 (&top)[L], u64& drop, u64 c) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const u64 hi = umax64(top[i], c);
        c = umin64(top[i], c);
        top[i] = hi;
    }
    drop = umax64(drop, c);
}

// The wave's `cnt` largest listed composites, descending, to out[0..cnt)
// (LDS, written by lane 0), zero padded up to a multiple of 8.  Returns, in
// every lane, the largest composite of the wave not extracted (a list's next
// head or anything a lane dropped), and in *n_out how many nonzero were
// extracted.  (The serial form: one wave-wide maximum per entry.)
template <int L>
__device__ inline u64 wave_extract_top_serial(u64 (&top)[L], u64 drop, int cnt, u64* out, int* n_out) {
    const int lane = threadIdx.x & (kWave - 1);
    int r = 0;
    for (; r < cnt; ++r) {
        const u64 wm = wave_max_u64(top[0]);
        if (wm == 0) break;  // wave-uniform
        if (lane == 0) out[r] = wm;
        if (top[0] == wm) {  // composites are unique: exactly one lane pops its head
#pragma unroll
            for (int i = 0; i + 1 < L; ++i) top[i] = top[i + 1];
            top[L - 1] = 0;
        }
    }
    *n_out = r;
    for (int j = r + lane; j < ((cnt + 7) & ~7); j += kWave) out[j] = 0;
    return umax64(wave_max_u64(top[0]), wave_max_u64(drop));
}

// At least `cnt` and at most cap = cnt rounded up to a multiple of 8 of the
// wave's largest listed composites, in no particular order, to out[0 ..)
// (LDS), zero padded up to cap; returns (every lane) the largest composite of
// the wave not written (a list entry below the threshold or anything a lane
// dropped) and in *n_out how many were written.  The entries written are
// those whose score word (high 32 bits) is at least a threshold found by a
// bitwise search from the top bit down: each probe counts the entries at or
// above it with one ballot per list position, and the search stops at the
// first probe whose count lies in [cnt, cap].  Scores tied on the whole word
// across that window take the serial form, and so does a small cnt (below
// kSearchMinCnt the serial form's cnt + 2 wave-wide maxima cost less than
// the probes: measured equal at cnt 5, the search 1 us faster at cnt 10).
// Every lane must call it.
constexpr int kSearchMinCnt = 8;
template <int L>
__device__ inline u64 wave_extract_top(u64 (&top)[L], u64 drop, int cnt, u64* out, int* n_out) {
    if (cnt < kSearchMinCnt) return wave_extract_top_serial(top, drop, cnt, out, n_out);
    const int lane = threadIdx.x & (kWave - 1);
    const int cap = (cnt + 7) & ~7;
    uint32_t hw[L];
#pragma unroll
    for (int i = 0; i < L; ++i) hw[i] = top[i] ? static_cast<uint32_t>(top[i] >> 32) : 0u;
    // entries at or above score word t (valid composites have a nonzero word)
    auto count_ge = [&](uint32_t t) -> int {
        int c = 0;
#pragma unroll
        for (int i = 0; i < L; ++i) c += __popcll(__ballot(hw[i] != 0u && hw[i] >= t));
        return c;
    };
    uint32_t thr = 0u;
    int c = count_ge(0u);
    if (c > cap) {
        // the largest t with count_ge(t) >= cnt, stopping early inside the window
        bool inside = false;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t t = thr | (1u << bit);
            const int ct = count_ge(t);
            if (ct >= cnt) {
                thr = t;
                c = ct;
                if (ct <= cap) {
                    inside = true;
                    break;
                }
            }
        }
        if (!inside) return wave_extract_top_serial(top, drop, cnt, out, n_out);
    }
    // compaction of the selected entries; each lane's largest unselected one
    int base = 0;
    u64 rest = drop;
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const bool sel = hw[i] != 0u && hw[i] >= thr;
        const u64 m = __ballot(sel);
        const u64 below = lane ? (m & (~0ull >> (64 - lane))) : 0ull;
        if (sel) out[base + __popcll(below)] = top[i];
        else rest = umax64(rest, top[i]);
        base += __popcll(m);
    }
    for (int j = base + lane; j < cap; j += kWave) out[j] = 0;
    *n_out = base;
    return wave_max_u64(rest);
}

// LDS scratch of block_top_m.
struct CandSmem {
    u64 wtop[16][kMaxCandM1];
    u64 wbound[16];
    int wcount[16];
};

// Workgroup candidate list from the lanes' lists: out[0..m) (global) = the m
// largest of the composites the waves extracted (each wave its mw largest),
// descending, zero padded; out[m] = a bound at least as large as every
// composite of the workgroup not in out[0..m).  mw <= m < kMaxCandM1; NW
// waves (blockDim.x == 64 NW, at most 16).  Every thread calls it, once per
// kernel.
template <int NW, int L>
__device__ inline void block_top_m(u64 (&top)[L], u64 drop, int m, int mw, u64* out, CandSmem& cs) {
    static_assert(NW >= 1 && NW <= 16, "at most 16 waves");
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    int cnt;
    const u64 bound = wave_extract_top(top, drop, mw, cs.wtop[wv], &cnt);
    if (lane == 0) {
        cs.wbound[wv] = bound;
        cs.wcount[wv] = cnt;
    }
    __syncthreads();
    // merge: an entry's rank is the number of larger entries over all lists
    // (unique values; the zero padding never counts).  Every lane reads the
    // same words (broadcasts): a run of 8 entries of every list is loaded at
    // once, one LDS round trip per run.
    u64 maxb = 0;
    int total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        maxb = umax64(maxb, cs.wbound[w]);
        total += cs.wcount[w];
    }
    const int mw8 = (mw + 7) & ~7;
    if (lane < cs.wcount[wv]) {
        const u64 x = cs.wtop[wv][lane];
        int rank = 0;
        for (int j0 = 0; j0 < mw8; j0 += 8) {
            u64 r[NW][8];
#pragma unroll
            for (int w = 0; w < NW; ++w)
#pragma unroll
                for (int j = 0; j < 8; ++j) r[w][j] = cs.wtop[w][j0 + j];
#pragma unroll
            for (int w = 0; w < NW; ++w)
#pragma unroll
                for (int j = 0; j < 8; ++j) rank += r[w][j] > x ? 1 : 0;
        }
        if (rank < m) out[rank] = x;
        else if (rank == m) out[m] = umax64(x, maxb);
    }
    if (wv == 0) {
        for (int j = total + lane; j < m; j += kWave) out[j] = 0;
        if (lane == 0 && total <= m) out[m] = maxb;
    }
}

// ---- register-resident sorted selection ----------------------------------------------

constexpr int kStageCap = 256;  // threshold-bin entries that are ranked in place

// Per-bin starts over a histogram in LDS, bins ordered from the top:
// start[b] = entries in bins > b.  Also finds, like block_threshold, the
// largest bin tb with suffix(tb) >= need (tb = -1 if total < need), with
// above = start[tb], at = cnt[tb], total = all entries; and zeroes cnt so it
// can serve as per-bin cursors.  The first kScanWaves waves do the scan, each
// lane a run of bins counted from the top (moved through registers with
// 16-byte LDS accesses), then lane prefixes and one exchange of the wave
// totals; the other waves only wait.  nbins <= 1 << kSelBits, a power of
// two; cnt and start 16-byte aligned; blockDim >= kScanWaves * 64.  Ends
// with a barrier.
constexpr int kScanWaves = 4;
__device__ inline void bin_starts(uint32_t* cnt, uint32_t* start, int nbins, uint32_t need, int& tb,
                                  uint32_t& above, uint32_t& at, uint32_t& total) {
    __shared__ uint32_t wsum[kScanWaves];
    __shared__ uint32_t res[4];
    constexpr int kLanes = kScanWaves * kWave;
    constexpr int kPer = (1 << kSelBits) / kLanes;  // bins per lane at full width
    static_assert(kPer % 4 == 0, "whole 16-byte groups of bins");
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int wv = t / kWave;
    const bool scanner = t < kLanes;
    const bool full = nbins == (1 << kSelBits);
    // this lane's run of bins [lo, hi), runs ordered from the top bin down
    const int per = full ? kPer : (nbins + kLanes - 1) / kLanes;
    const int hi = scanner ? max(nbins - per * t, 0) : 0;
    const int lo = max(hi - per, 0);
    uint4 q[kPer / 4];
    uint32_t mine = 0;
    if (scanner) {
        if (full) {
#pragma unroll
            for (int j = 0; j < kPer / 4; ++j) {
                q[j] = *reinterpret_cast<const uint4*>(cnt + lo + 4 * j);
                mine += q[j].x + q[j].y + q[j].z + q[j].w;
            }
        } else {
            for (int b = lo; b < hi; ++b) mine += cnt[b];
        }
    }
    uint32_t pre = mine, sum = mine;
    if (wv < kScanWaves) {
#define CSA_SCAN_STEP(o)                                         \
        {                                                        \
            const uint32_t other = xor_lanes<o>(sum);            \
            if (lane & (o)) pre += other;                        \
            sum += other;                                        \
        }
        CSA_SCAN_STEP(1) CSA_SCAN_STEP(2) CSA_SCAN_STEP(4) CSA_SCAN_STEP(8) CSA_SCAN_STEP(16) CSA_SCAN_STEP(32)
#undef CSA_SCAN_STEP
        if (lane == 0) wsum[wv] = sum;
    }
    __syncthreads();
    if (wv < kScanWaves) {
        uint32_t tot = 0, before = 0;
#pragma unroll
        for (int w = 0; w < kScanWaves; ++w) {
            const uint32_t x = wsum[w];
            tot += x;
            before += w < wv ? x : 0u;
        }
        uint32_t acc = before + pre - mine;  // entries in bins >= hi
        int found = -1;
        uint32_t f_above = 0, f_at = 0;
        auto visit = [&](uint32_t c, int b) -> uint32_t {
            const uint32_t s0 = acc;
            if (tot >= need && acc < need && acc + c >= need) {
                found = b;
                f_above = acc;
                f_at = c;
            }
            acc += c;
            return s0;
        };
        if (full) {
            uint4 st[kPer / 4];
#pragma unroll
            for (int j = kPer / 4 - 1; j >= 0; --j) {  // from the run's top bin down
                st[j].w = visit(q[j].w, lo + 4 * j + 3);
                st[j].z = visit(q[j].z, lo + 4 * j + 2);
                st[j].y = visit(q[j].y, lo + 4 * j + 1);
                st[j].x = visit(q[j].x, lo + 4 * j);
            }
#pragma unroll
            for (int j = 0; j < kPer / 4; ++j) {
                *reinterpret_cast<uint4*>(start + lo + 4 * j) = st[j];
                *reinterpret_cast<uint4*>(cnt + lo + 4 * j) = make_uint4(0, 0, 0, 0);
            }
        } else {
            for (int b = hi - 1; b >= lo; --b) {
                start[b] = visit(cnt[b], b);
                cnt[b] = 0;
            }
        }
        if (found >= 0) {
            res[0] = static_cast<uint32_t>(found);
            res[1] = f_above;
            res[2] = f_at;
        }
        if (t == 0) {
            res[3] = tot;
            if (tot < need) {
                res[0] = 0xffffffffu;
                res[1] = tot;
                res[2] = 0;
            }
        }
    }
    __syncthreads();
    tb = static_cast<int>(res[0]);
    above = res[1];
    at = res[2];
    total = res[3];
}

// LDS scratch of select_sorted.
struct SortSmem {
    uint32_t cnt[1 << kSelBits];
    uint32_t start[1 << kSelBits];
};

// Outcome of select_first_pass.
struct FirstPass {
    uint32_t total;    // live entries
    uint32_t written;  // indices written (when done)
    bool done;
    // otherwise the threshold bin's entries wait in pool[0..np): the rest of
    // the selection is the `need` largest of them, written from out[off] on,
    // with digits from bit pb
    uint32_t np, off, need;
    int pb;
};

// The first pass of select_sorted taken straight from registers: the
// threads' v[] hold the live entries (zero = none), all sharing their top pb
// bits; ss.cnt must be zero over its 1 << kSelBits bins, visible to every
// thread.  Writes the indices of every entry that the pass places (the bins
// above the threshold bin, and that bin too when it holds at most kStageCap
// entries) to their final positions in out.  If the threshold bin is larger,
// its entries are compacted into pool for select_sorted to finish.  Every
// thread calls it; the result is the same in every thread.
template <int V>
__device__ inline FirstPass select_first_pass(u64 (&v)[V], uint32_t need, int pb, int* out, u64* stage, SortSmem& ss,
                                              u64* pool, uint32_t* n_pool) {
    const int db = min(kSelBits, 64 - pb);
    const int nb = 1 << db;
    const int shift = 64 - pb - db;
    const u64 dmask = static_cast<u64>(nb - 1);
#pragma unroll
    for (int u = 0; u < V; ++u)
        if (v[u]) atomicAdd(&ss.cnt[(v[u] >> shift) & dmask], 1u);
    __syncthreads();
    int td;
    uint32_t above, at, total;
    bin_starts(ss.cnt, ss.start, nb, need, td, above, at, total);
    const bool all = td < 0;
    const bool stage_td = !all && at <= static_cast<uint32_t>(kStageCap);
    int dg[V];
#pragma unroll
    for (int u = 0; u < V; ++u) {
        dg[u] = v[u] ? static_cast<int>((v[u] >> shift) & dmask) : -1;
        if (dg[u] >= 0 && (all || dg[u] > td || (dg[u] == td && stage_td)))
            stage[ss.start[dg[u]] + atomicAdd(&ss.cnt[dg[u]], 1u)] = v[u];
    }
    if (threadIdx.x == 0) *n_pool = 0;
    __syncthreads();
    const uint32_t nst = all ? total : above + (stage_td ? at : 0u);
    for (uint32_t i = threadIdx.x; i < nst; i += blockDim.x) {
        const u64 x = stage[i];
        const int d = static_cast<int>((x >> shift) & dmask);
        const uint32_t s0 = ss.start[d];
        const uint32_t c = ss.cnt[d];
        uint32_t r = 0;
        for (uint32_t j = 0; j < c; ++j) r += stage[s0 + j] > x ? 1u : 0u;
        if (all || d > td || r < need - above) out[s0 + r] = composite_index(x);
    }
    FirstPass fp{};
    fp.total = total;
    if (all || stage_td) {
        fp.done = true;
        fp.written = all ? total : need;
        return fp;
    }
#pragma unroll
    for (int u = 0; u < V; ++u) {
        const bool keep = dg[u] == td;
        const uint32_t p = wave_append_pos(keep, n_pool);
        if (keep) pool[p] = v[u];
    }
    __syncthreads();
    fp.done = false;
    fp.np = at;
    fp.off = above;
    fp.need = need - above;
    fp.pb = pb + db;
    return fp;
}

// The `need` largest of the unique nonzero composites pool[0..np) (LDS),
// written sorted descending as indices to out[0 ..) (global); all of them if
// there are fewer.  Returns how many were written.  Every entry must share
// its top pb bits with the others.
//
// Each pass histograms the kSelBits-wide digit after those pb bits.  The
// bins' starts place every entry of the bins above the threshold bin (and of
// the threshold bin itself when it holds at most kStageCap entries) at its
// final position: entries are staged bin by bin, then each is ranked inside
// its bin.  A larger threshold bin is compacted to the front of the pool and
// goes on to the next digit alone.  np <= kPoolRegs * blockDim.x; stage
// holds kTopkMaxK + kStageCap composites; *n_pool is a spare LDS counter.
// Every thread calls it; pool is consumed.
template <int kPoolRegs>
__device__ inline uint32_t select_sorted(u64* pool, uint32_t np, uint32_t need, int pb, int* out, u64* stage,
                                         SortSmem& ss, uint32_t* n_pool) {
    uint32_t off = 0;
    while (true) {
        const int db = min(kSelBits, 64 - pb);
        const int nb = 1 << db;
        const int shift = 64 - pb - db;
        const u64 dmask = static_cast<u64>(nb - 1);
        for (int i = threadIdx.x; i < nb; i += blockDim.x) ss.cnt[i] = 0;
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < np; i += blockDim.x)
            atomicAdd(&ss.cnt[(pool[i] >> shift) & dmask], 1u);
        __syncthreads();
        int td;
        uint32_t above, at, total;
        bin_starts(ss.cnt, ss.start, nb, need, td, above, at, total);
        const bool all = td < 0;
        const bool stage_td = !all && at <= static_cast<uint32_t>(kStageCap);
        for (uint32_t i = threadIdx.x; i < np; i += blockDim.x) {
            const u64 x = pool[i];
            const int d = static_cast<int>((x >> shift) & dmask);
            if (all || d > td || (d == td && stage_td)) stage[ss.start[d] + atomicAdd(&ss.cnt[d], 1u)] = x;
        }
        __syncthreads();
        const uint32_t nst = all ? total : above + (stage_td ? at : 0u);
        for (uint32_t i = threadIdx.x; i < nst; i += blockDim.x) {
            const u64 x = stage[i];
            const int d = static_cast<int>((x >> shift) & dmask);
            const uint32_t s = ss.start[d];
            const uint32_t c = ss.cnt[d];
            uint32_t r = 0;
            for (uint32_t j = 0; j < c; ++j) r += stage[s + j] > x ? 1u : 0u;
            if (all || d > td || r < need - above) out[off + s + r] = composite_index(x);
        }
        if (all) return off + total;
        if (stage_td) return off + need;
        // the threshold bin alone goes on with the next digit
        u64 keep[kPoolRegs];
#pragma unroll
        for (int u = 0; u < kPoolRegs; ++u) {
            const uint32_t i = threadIdx.x + u * blockDim.x;
            const u64 x = i < np ? pool[i] : 0ull;
            keep[u] = (i < np && static_cast<int>((x >> shift) & dmask) == td) ? x : 0ull;
        }
        if (threadIdx.x == 0) *n_pool = 0;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kPoolRegs; ++u) {
            const uint32_t p = wave_append_pos(keep[u] != 0, n_pool);
            if (keep[u]) pool[p] = keep[u];
        }
        __syncthreads();
        np = at;
        off += above;
        need -= above;
        pb += db;
    }
}

}  // namespace csa

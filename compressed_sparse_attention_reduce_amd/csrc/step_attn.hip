// Fused top-k + partial attention of the bf16 decode step.
//
// Cross-workgroup synchronisation inside a kernel costs a device-scope
// fence per workgroup on this chip (tens of microseconds for a grid of this
// size), so instead of a separate top-k launch feeding the attention, every
// attention workgroup computes the same (deterministic) top k of its
// sequence from the per-slot candidate lists into LDS, then attends over its
// split of the selected rows plus the SWA window.  Workgroup (0, 0) of each
// sequence also writes topk_idx and topk_count.  Top-k: topk.hip (page 1,
// ARCHITECTURE_AND_MEMORY_AUDIT.md F3); attention: attn.hip (page 1, fmha
// sink correction).  The split partials are merged by k_attn_merge.
#include "attn_split.h"
#include "topk_final.h"

namespace csa {

namespace {

__host__ __device__ inline size_t topk_attn_lds_bytes() {
    return sizeof(FinalSmem) + sizeof(int) * kTopkMaxK;
}

__global__ __launch_bounds__(kFinalThreads) void k_topk_attn(TopkArgs ta, CandArgs c, AttnArgs a, int n_splits) {
    if (a.dev) {  // counters on the device: the step's view of them after its jobs
        const DevState st = dev_load(a.dev, a.w, a.max_comp);
        if (a.dev_pos && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) *a.dev_pos = st.pos;
        const int n = st.n_comp + (dev_completes(st, a.m, a.max_comp) ? 1 : 0);
        ta.n = n;
        a.n_comp = n;
        a.swa_head = (st.swa_head + 1) % a.w;
        a.swa_len = st.swa_len + 1 < a.w ? st.swa_len + 1 : a.w;
    }
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    FinalSmem& fs = *reinterpret_cast<FinalSmem*>(smem);
    int* sidx = reinterpret_cast<int*>(smem + sizeof(FinalSmem));  // this sequence's top-k indices
    const int split = blockIdx.x;
    const int hg = blockIdx.y;
    const int b = blockIdx.z;
    uint4 qv[AttnSplit<kFinalThreads>::kQBatch];
    attn_load_q<kFinalThreads>(a, hg, b, qv);
    // the top k of sequence b (one query row each)
    uint32_t k_eff = 0;
    const bool done = c.lists && union_topk(fs, c, b, ta.k, sidx, k_eff);
    if (!done) {
        __syncthreads();  // the fast path's reads of LDS are over
        k_eff = exact_row_topk(fs, score_row(ta, b), ta.n, ta.k, sidx);
    }
    __syncthreads();  // sidx complete; the top-k LDS is free for the attention
    if (split == 0 && hg == 0) {
        int* out = ta.idx + static_cast<long long>(b) * ta.k;
        for (int j = threadIdx.x; j < ta.k; j += kFinalThreads) out[j] = j < static_cast<int>(k_eff) ? sidx[j] : -1;
        if (ta.count && threadIdx.x == 0) ta.count[b] = static_cast<int>(k_eff);
    }
    attn_split<kFinalThreads>(a, n_splits, split, hg, b, sidx, static_cast<int>(k_eff), qv,
                              reinterpret_cast<uint16_t*>(smem));
}

static_assert(sizeof(FinalSmem) >= sizeof(uint16_t) * ((kR + kHeadGroup) * (512 + 8) + kHeadGroup * kPPitch),
              "the attention split fits in the top-k LDS at d = 512");

}  // namespace

int topk_attn_workgroups(int batch, int h, int n_max) { return attn_splits(n_max) * (h / kHeadGroup) * batch; }

hipError_t launch_topk_attn(const TopkArgs& ta, const CandArgs* cands, AttnArgs a, hipStream_t s) {
    if (ta.t != 1 || a.d > 512 || a.batch != ta.batch) return hipErrorInvalidValue;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    static bool opted_in[64] = {};
    if (!opted_in[dev]) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_topk_attn),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(topk_attn_lds_bytes()));
        if (e != hipSuccess) return e;
        opted_in[dev] = true;
    }
    const int ns = attn_splits(a.n_max);
    a.ws_o = static_cast<float*>(a.ws);
    a.ws_ml = a.ws_o + static_cast<size_t>(a.batch) * a.h * ns * a.d;
    const CandArgs c = cands ? *cands : CandArgs{nullptr, 0, 0, 0};
    hipLaunchKernelGGL(k_topk_attn, dim3(ns, a.h / kHeadGroup, a.batch), dim3(kFinalThreads), topk_attn_lds_bytes(),
                       s, ta, c, a, ns);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_attn_merge(a, ns, s);
}

}  // namespace csa

// The epilogue of one 64-head x 16-key tile of the lightning-indexer score,
// shared by every bf16 scan so that they all produce the same bits for the
// same (query, key) pair.
//
// Page 1, ARCHITECTURE_AND_MEMORY_AUDIT.md, finding F3 (paper section 2.3.1,
// eq. 16): I[s] = sum_h w[h] * ReLU(q[h] . K[s]).
#pragma once

#include "common.h"

namespace csa {

namespace {

// acc[mt]: the 16x16 v_mfma_f32_16x16x32_bf16 accumulator of head tile mt
// (register r of lane (lg, li) <-> head 16*mt + 4*lg + r, key li); wr holds
// the matching head weights.  Returns the score of key li in every lane:
// ReLU and weight per head in registers (fixed order: mt, then r), then the
// four lane groups summed by two lane swaps.
__device__ __forceinline__ float tile_head_sum(const f32x4 (&acc)[4], const float (&wr)[4][4]) {
    float part = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) part += wr[mt][r] * fmaxf(acc[mt][r], 0.f);
    part += xor_lanes_f32<16>(part);
    part += xor_lanes_f32<32>(part);
    return part;
}

}  // namespace

}  // namespace csa

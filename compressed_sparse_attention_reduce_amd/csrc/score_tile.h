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

// ReLU of a finite float in one instruction: the median of (x, 0, FLT_MAX)
// is max(x, 0) for every finite x (fmaxf would first quiet a possible NaN
// with a second instruction; inputs here are finite by contract).
__device__ __forceinline__ float relu_finite(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, 3.402823466e38f); }

// acc[mt]: the 16x16 v_mfma_f32_16x16x32_bf16 accumulator of head tile mt
// (register r of lane (lg, li) <-> head 16*mt + 4*lg + r, key li); wr holds
// the matching head weights.  The lane's share of the score of key li: ReLU
// and weight per head in registers — one running sum per head tile (in the
// order r = 0..3), the four tile sums added pairwise, so the dependent chain
// is 6 deep, not 16.
__device__ __forceinline__ float tile_lane_part(const f32x4 (&acc)[4], const float (&wr)[4][4]) {
    float p[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        p[mt] = wr[mt][0] * relu_finite(acc[mt][0]);
#pragma unroll
        for (int r = 1; r < 4; ++r) p[mt] += wr[mt][r] * relu_finite(acc[mt][r]);
    }
    return (p[0] + p[1]) + (p[2] + p[3]);
}

// The score of key li in every lane: the four lane groups' shares summed by
// two lane swaps, as (row 0 + row 1) + (row 2 + row 3).
__device__ __forceinline__ float tile_head_sum(const f32x4 (&acc)[4], const float (&wr)[4][4]) {
    float part = tile_lane_part(acc, wr);
    part += xor_lanes_f32<16>(part);
    part += xor_lanes_f32<32>(part);
    return part;
}

// Two query rows at once with the same additions as tile_head_sum: one
// 16-lane swap exchanges the rows' shares (lanes of rows 0 and 2 keep row
// a's pair sums, rows 1 and 3 row b's), one 32-lane swap finishes both.
// Lanes with (lane & 16) == 0 return row a's score of key li, the others
// row b's.
__device__ __forceinline__ float tile_head_sum2(const f32x4 (&acc_a)[4], const float (&wr_a)[4][4],
                                                const f32x4 (&acc_b)[4], const float (&wr_b)[4][4]) {
    const float pa = tile_lane_part(acc_a, wr_a);
    const float pb = tile_lane_part(acc_b, wr_b);
    // [0] = rows (a0, b0, a2, b2), [1] = rows (a1, b1, a3, b3)
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(pa), __float_as_uint(pb), false, false);
    const float r0 = __uint_as_float(static_cast<uint32_t>(r[0]));
    const float r1 = __uint_as_float(static_cast<uint32_t>(r[1]));
    const float s = r0 + r1;
    // [0] = low half twice, [1] = high half twice
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    const float h0 = __uint_as_float(static_cast<uint32_t>(h[0]));
    const float h1 = __uint_as_float(static_cast<uint32_t>(h[1]));
    return h0 + h1;
}

}  // namespace

}  // namespace csa

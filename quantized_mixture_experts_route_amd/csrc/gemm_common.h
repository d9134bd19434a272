// gemm_common.h -- pieces shared by the prefill and decode projection kernels.
//
// MFMA operand mapping (v_mfma_f32_16x16x32_{f16,bf16}): lane l = 16*g + c
// supplies row c of the A block and column c of the B block, each as 8
// values at the same 8 positions of the 32-long contraction, chosen by the
// lane group g.  The contraction is indifferent to which physical inputs
// those 32 positions are, as long as A and B use the same ones.  So within a
// K super-step of 128 inputs, lane group g takes the 32 consecutive inputs
// [32g, 32g+32) -- one contiguous span of packed codes per lane (16 B at
// 4 bits) -- and MFMA step t (0..3) consumes inputs [32g+8t, 32g+8t+8).
// The result block D[16x16] lands with lane l holding rows 4g..4g+3 of
// column c.
#pragma once

#include "qmoe_device.h"
#include "qmoe_internal.h"

namespace qmoe {

struct WeightRow {
    const uint8_t* codes;
    const uint16_t* scales;
    const uint8_t* zp;  // nullable
};

__device__ inline WeightRow weight_row(const ProjArgs& w, int64_t row, int K, int block_size)
{
    const int n_blocks = K / block_size;
    WeightRow r;
    r.codes = w.codes + row * (int64_t)(K * w.bits / 8);
    r.scales = reinterpret_cast<const uint16_t*>(w.scales) + row * n_blocks;
    r.zp = w.zp ? w.zp + row * zp_row_bytes(n_blocks, w.bits) : nullptr;
    return r;
}

// B fragment for MFMA step t of a span whose step-t group starts at input kk.
template <int DT, int BITS>
__device__ inline u32x4 b_fragment(const Span<BITS>& sp, int t, int kk, const WeightRow& r,
                                   float zp_fallback, int block_size)
{
    const int blk = kk / block_size;
    const float scale = Dt<DT>::to_float(r.scales[blk]);
    const float zp = zero_point<BITS>(r.zp, blk, zp_fallback);
    return dequant8<DT, BITS>(span_group<BITS>(sp, t), zp, scale);
}

template <int DT>
__device__ inline float act_value(int act, float gate, float up)
{
    return act == kGeGLU ? gated<kGeGLU>(gate, up) : gated<kSwiGLU>(gate, up);
}

}  // namespace qmoe

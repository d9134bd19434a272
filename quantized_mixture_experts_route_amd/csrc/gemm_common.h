// gemm_common.h -- pieces shared by the prefill and decode projection kernels.
//
// MFMA operand mapping (v_mfma_f32_16x16x32_{f16,bf16}): lane l = 16*g + c
// supplies row c of the A block and column c of the B block, each as 8
// values at the same 8 positions of the 32-long contraction, chosen by the
// lane group g.  The contraction is indifferent to which physical inputs
// those 32 positions are, as long as A and B use the same ones.  So within a
// K super-step of 128 inputs, lane group g takes the 32 consecutive inputs
// [32g, 32g+32) -- one contiguous span of packed codes per lane (16 B at
// 4 bits) -- and MFMA step t (0..3) consumes 8 of them in the register order
// code_order<DT, BITS>() (qmoe_device.h); the A values are permuted to the
// same order.  The result block D[16x16] lands with lane l holding rows
// 4g..4g+3 of column c.
#pragma once

#include "qmoe_device.h"
#include "qmoe_internal.h"

namespace qmoe {

struct WeightRow {
    const uint8_t* codes;
    const uint16_t* scales;
    const uint8_t* zp;  // nullable
    int bits;

    // byte of the zero-point row holding block blk's value
    __device__ uint32_t zp_byte(int blk) const { return zp[bits == 3 ? blk : blk / (8 / bits)]; }
};

__device__ inline WeightRow weight_row(const ProjArgs& w, int64_t row, int K, int block_size)
{
    const int n_blocks = K / block_size;
    WeightRow r;
    r.codes = w.codes + row * (int64_t)(K * w.bits / 8);
    r.scales = reinterpret_cast<const uint16_t*>(w.scales) + row * n_blocks;
    r.zp = w.zp ? w.zp + row * zp_row_bytes(n_blocks, w.bits) : nullptr;
    r.bits = w.bits;
    return r;
}

// Zero-point handling of a projection, fixed per launch:
//   kZpConst   one zero point for every block (offset or centre), a multiple of
//              1/2 below 256: fast dequant
//   kZpTensor  per-block uint8 zero points (integers): fast dequant
//   kZpGeneric one zero point of any other value: float32 dequant
enum : int { kZpConst = 0, kZpTensor = 1, kZpGeneric = 2 };

// Raw bits of one block's scale and packed zero point, loaded ahead of use so
// that no load waits on another.
struct RawParams {
    uint32_t scale;
    uint32_t zp;
    int blk;
};

template <int ZP>
__device__ inline RawParams load_params(const WeightRow& r, int kk, int block_size)
{
    RawParams q;
    q.blk = kk >> __builtin_ctz((unsigned)block_size);  // block_size is a power of two
    q.scale = r.scales[q.blk];
    q.zp = 0;
    if constexpr (ZP == kZpTensor) q.zp = r.zp_byte(q.blk);
    return q;
}

struct BlockParams {
    float zp;
    float scale;
};

template <int DT, int BITS, int ZP>
__device__ inline BlockParams decode_params(const RawParams& q, float zp_const)
{
    BlockParams b;
    b.scale = Dt<DT>::to_float((uint16_t)q.scale);
    if constexpr (ZP == kZpTensor) {
        if constexpr (BITS == 3) {
            b.zp = (float)q.zp;
        } else {
            constexpr int per = 8 / BITS;
            b.zp = (float)((q.zp >> ((q.blk % per) * BITS)) & ((1u << BITS) - 1u));
        }
    } else {
        b.zp = zp_const;
    }
    return b;
}

template <int DT, int BITS, int ZP>
__device__ inline u32x4 dequant_zp(const Span<BITS>& sp, int t, const BlockParams& b)
{
    if constexpr (ZP == kZpGeneric) return dequant_step_generic<DT, BITS>(sp, t, b.zp, b.scale);
    else return dequant_step<DT, BITS, ZP == kZpTensor>(sp, t, b.zp, b.scale);
}

inline int zp_mode(const ProjArgs& w)
{
    return w.zp ? kZpTensor : (w.fast ? kZpConst : kZpGeneric);
}

// 32 consecutive dtype values of an A row starting at element k (16-byte aligned).
__device__ inline void load_a_span(const uint16_t* row, int k, uint32_t (&v)[16])
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(row + k + 8 * q);
        v[4 * q + 0] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
    }
}

// SwiGLU with the operator's parameters [qmoe.rs, swiglu_value]: the gate
// bounded above by limit (fminf), the linear part clamped to [-limit, limit]
// unless NaN, then g * sigmoid(alpha g) * (u + beta).  alpha = 1, beta = 0,
// limit = +inf give silu(g) * u.  GeGLU takes no parameters.
template <int DT>
__device__ inline float act_value(int act, float gate, float up, const ActParams& ap)
{
    if (act == kGeGLU) return gated<kGeGLU>(gate, up);
    const float g = fminf(gate, ap.limit);
    const float u = isnan(up) ? up : fminf(fmaxf(up, -ap.limit), ap.limit);
    return g * sigmoid_fast(ap.alpha * g) * (u + ap.beta);
}

// fc1 (+ fc3) weight row of a gate or up row of activation column j, by the
// gate/up layout [qmoe.rs, swiglu_fusion]: 1 interleaved (gate 2j, up 2j+1),
// 2 halves (gate j, up I + j), 0 a separate fc3 (gate j of fc1, up j of fc3).
__device__ inline int64_t fc1_row(int fusion, int j, bool up, int I)
{
    if (fusion == 1) return 2 * (int64_t)j + (up ? 1 : 0);
    return (int64_t)j + (fusion == 2 && up ? I : 0);
}

// fc2 row values of a decode launch that folds the combine in are written
// with device-scope (write-through) stores, so another XCD's combining
// workgroup reads them from the device coherence point without any L2
// writeback or invalidation.
__device__ inline void store_y2(float* dst, float v, bool through)
{
    if (through) __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *dst = v;
}

// Arrival of one workgroup on fc2 column block n (every thread calls it, with
// the workgroup's fc2 rows of the block already stored through store_y2, or
// none at all); the last of `expected` arrivals combines columns
// [c0, c0 + width) of every token: out[t, c] = RNE_dtype(sum over slots s in
// order of w[t, s] * y2[t*top_k + s, c]) [qmoe.rs, qmoe_combine:
// slot-ordered float32 sum, rounded once].  Ordering: each wave waits for its
// own device-scope stores to complete (s_waitcnt) before the workgroup's
// arrival increments the counter, and the last arrival reads y2 with
// device-scope loads after its increment has returned.
template <int DT>
__device__ inline void fc2_arrive_combine(const FusedCombine& fc, const float* y2, int H, int top_k,
                                          int n, int c0, int width, int expected)
{
    __shared__ int s_last;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        s_last = __hip_atomic_fetch_add(&fc.counters[n], 1, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == expected - 1;
    }
    __syncthreads();
    if (!s_last) return;
    uint16_t* out = reinterpret_cast<uint16_t*>(fc.out);
    const int items = fc.T * width;
    for (int i = threadIdx.x; i < items; i += blockDim.x) {
        const int t = i / width;
        const int c = c0 + (i - t * width);
        float sum = 0.0f;
        for (int s = 0; s < top_k; ++s) {
            const int64_t r = (int64_t)t * top_k + s;
            sum += fc.weights[r] *
                   __hip_atomic_load(y2 + r * H + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        out[(int64_t)t * H + c] = Dt<DT>::from_float(sum);
    }
    if (threadIdx.x == 0) {
        __hip_atomic_store(&fc.counters[n], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace qmoe

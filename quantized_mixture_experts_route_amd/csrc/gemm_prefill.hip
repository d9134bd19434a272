// gemm_prefill.hip -- grouped projection for many routed rows per expert.
//
// One workgroup (4 wavefronts) takes one work-list item {expert, m, n}: up to
// kPrefillMT routed rows of that expert against 256 weight rows, each
// wavefront owning 64 weight rows (4 MFMA column blocks of 16) for all the
// item's rows.  Packed codes stream from HBM straight into registers, are
// dequantized there as (code - zp) * scale and fed to bf16/fp16 MFMA; the
// A rows (gathered hidden states for fc1, sorted activations for fc2) are
// staged once per K super-step in LDS and shared by the four wavefronts.
// [PR 32198: weights stay packed in HBM and are dequantized in registers
// inside the GEMM; gemm_quant_moe.rs, moe_fp8_grouped_gemm: workgroups stride
// over a compacted work-list, rows addressed through sorted route ids.]
//
// fc1 (+ activation): a wavefront's 4 column blocks are the gate rows 2j and
// the up rows 2j+1 of 32 activation columns, arranged so that gate and up of
// one column land in the same lane and accumulator slot; the epilogue
// applies SwiGLU/GeGLU and writes the activation, rounded to the dtype, at
// the route's sorted position.  fc2: the epilogue writes float32 results at
// the route id's row of y2.
#include "gemm_common.h"

namespace qmoe {
namespace {

constexpr int kThreads = 256;
constexpr int kLda = kSuperK + 8;  // LDS row pitch in 16-bit elements

template <int DT, int BITS, bool FC1, int MT>
__global__ __launch_bounds__(kThreads) void prefill_kernel(ProjLaunch p)
{
    constexpr int MB = MT / 16;
    __shared__ __attribute__((aligned(16))) uint16_t a_lds[MT * kLda];
    __shared__ int row_src[MT];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int c = lane & 15;
    const int K = p.K;
    const int n_items = *p.n_items;
    const uint16_t* a_src = reinterpret_cast<const uint16_t*>(p.a);

    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int e = p.worklist[3 * item + 0];
        const int mt = p.worklist[3 * item + 1];
        const int nt = p.worklist[3 * item + 2];
        const int row0 = p.offsets[e] + mt * MT;
        const int rows = min(MT, p.offsets[e + 1] - row0);

        int col0;  // fc1: first activation column of this wave; fc2: first hidden column
        bool active;
        int64_t wrow[4];
        if constexpr (FC1) {
            col0 = nt * kPrefillFc1Cols + wave * 32;
            active = col0 < p.N / 2;
            wrow[0] = 2 * (col0 + c);
            wrow[1] = 2 * (col0 + c) + 1;
            wrow[2] = 2 * (col0 + 16 + c);
            wrow[3] = 2 * (col0 + 16 + c) + 1;
        } else {
            col0 = nt * kPrefillFc2Cols + wave * 64;
            active = col0 < p.N;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) wrow[nb] = col0 + nb * 16 + c;
        }
        WeightRow wr[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            wr[nb] = weight_row(p.w, (int64_t)e * p.N + (active ? wrow[nb] : 0), K, p.block_size);
        }

        __syncthreads();  // the previous item is done with row_src and a_lds
        for (int i = tid; i < MT; i += kThreads) {
            int src = -1;
            if (i < rows) src = FC1 ? p.sorted[row0 + i] / p.top_k : row0 + i;
            row_src[i] = src;
        }
        __syncthreads();

        f32x4 acc[MB][4];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int k0 = 0; k0 < K; k0 += kSuperK) {
#pragma unroll
            for (int q = tid; q < MT * 16; q += kThreads) {
                const int i = q >> 4;
                const int ch = q & 15;
                const int src = row_src[i];
                u32x4 v = {0u, 0u, 0u, 0u};
                if (src >= 0) {
                    v = *reinterpret_cast<const u32x4*>(a_src + (int64_t)src * K + k0 + ch * 8);
                }
                *reinterpret_cast<u32x4*>(&a_lds[i * kLda + ch * 8]) = v;
            }
            Span<BITS> sp[4];
            if (active) {
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) sp[nb] = load_span<BITS>(wr[nb].codes, k0 + 32 * g);
            }
            __syncthreads();
            if (active) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int kk = k0 + 32 * g + 8 * t;
                    u32x4 bf[4];
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb) {
                        bf[nb] = b_fragment<DT, BITS>(sp[nb], t, kk, wr[nb], p.w.zp_fallback,
                                                      p.block_size);
                    }
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        if (mb * 16 < rows) {
                            const u32x4 af = *reinterpret_cast<const u32x4*>(
                                &a_lds[(mb * 16 + c) * kLda + 32 * g + 8 * t]);
#pragma unroll
                            for (int nb = 0; nb < 4; ++nb) {
                                acc[mb][nb] = Dt<DT>::mfma(af, bf[nb], acc[mb][nb]);
                            }
                        }
                    }
                }
            }
            __syncthreads();
        }

        if (!active) continue;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = mb * 16 + 4 * g + i;
                if (m >= rows) continue;
                if constexpr (FC1) {
                    const int I = p.N / 2;
                    uint16_t* out = reinterpret_cast<uint16_t*>(p.act_out) + (int64_t)(row0 + m) * I;
                    out[col0 + c] = Dt<DT>::from_float(act_value<DT>(p.act, acc[mb][0][i], acc[mb][1][i]));
                    out[col0 + 16 + c] =
                        Dt<DT>::from_float(act_value<DT>(p.act, acc[mb][2][i], acc[mb][3][i]));
                } else {
                    float* out = p.y2 + (int64_t)p.sorted[row0 + m] * p.N;
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb) out[col0 + nb * 16 + c] = acc[mb][nb][i];
                }
            }
        }
    }
}

template <bool FC1, int DT>
hipError_t launch_dt(const ProjLaunch& p, hipStream_t s)
{
    const dim3 grid((unsigned)p.grid), block(kThreads);
    switch (p.w.bits) {
    case 2: hipLaunchKernelGGL((prefill_kernel<DT, 2, FC1, kPrefillMT>), grid, block, 0, s, p); break;
    case 3: hipLaunchKernelGGL((prefill_kernel<DT, 3, FC1, kPrefillMT>), grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<DT, 4, FC1, kPrefillMT>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fc1_prefill(const ProjLaunch& p, int dtype, hipStream_t s)
{
    return dtype == kBF16 ? launch_dt<true, kBF16>(p, s) : launch_dt<true, kF16>(p, s);
}

hipError_t launch_fc2_prefill(const ProjLaunch& p, int dtype, hipStream_t s)
{
    return dtype == kBF16 ? launch_dt<false, kBF16>(p, s) : launch_dt<false, kF16>(p, s);
}

}  // namespace qmoe

// gemm_prefill.hip -- grouped projection for many routed rows per expert.
//
// One workgroup (4 wavefronts) takes one work-list item {expert, m, n}: up to
// kPrefillMT routed rows of that expert against 256 weight rows, each
// wavefront owning 64 weight rows (4 MFMA column blocks of 16) for all the
// item's rows.  Packed codes stream from HBM straight into registers, are
// dequantized there as (code - zp) * scale and fed to bf16/fp16 MFMA; the
// A rows (gathered hidden states for fc1, sorted activations for fc2) are
// staged per K super-step in a double-buffered LDS tile shared by the four
// wavefronts, already permuted to the MFMA register order, while the next
// super-step's A rows and packed spans are in flight.
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
constexpr int kPitch = kSuperK / 2 + 4;  // LDS row pitch in 32-bit words (64 data + 4 pad)

template <int DT, int BITS, bool FC1, int MT, int ZP>
__global__ __launch_bounds__(kThreads) void prefill_kernel(ProjLaunch p)
{
    constexpr Order O = code_order<DT, BITS>();
    constexpr int MB = MT / 16;
    constexpr int kChunks = MT * 4 / kThreads;  // (row, lane-group span) pieces staged per thread
    __shared__ __attribute__((aligned(16))) uint32_t a_lds[2][MT * kPitch];
    __shared__ int row_src[MT];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int c = lane & 15;
    const int K = p.K;
    const int n_super = K / kSuperK;
    const int n_items = *p.n_items;
    const bool two_blocks = p.block_size < 32;
    const uint16_t* a_src = reinterpret_cast<const uint16_t*>(p.a);

    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int e = p.worklist[3 * item + 0];
        const int mt = p.worklist[3 * item + 1];
        const int nt = p.worklist[3 * item + 2];
        const int row0 = p.offsets[e] + mt * MT;
        const int rows = min(MT, p.offsets[e + 1] - row0);

        int col0;  // fc1: first activation column of this wave; fc2: first hidden column
        bool active;
        WeightRow wr[4];
        if constexpr (FC1) {
            col0 = nt * kPrefillFc1Cols + wave * 32;
            active = col0 < p.N / 2;
            const int64_t base = (int64_t)e * p.N + (active ? 2 * (col0 + c) : 0);
            wr[0] = weight_row(p.w, base, K, p.block_size);
            wr[1] = weight_row(p.w, base + 1, K, p.block_size);
            wr[2] = weight_row(p.w, base + (active ? 32 : 0), K, p.block_size);
            wr[3] = weight_row(p.w, base + (active ? 33 : 1), K, p.block_size);
        } else {
            col0 = nt * kPrefillFc2Cols + wave * 64;
            active = col0 < p.N;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                wr[nb] = weight_row(p.w, (int64_t)e * p.N + (active ? col0 + nb * 16 + c : 0), K,
                                    p.block_size);
            }
        }

        __syncthreads();  // the previous item is done with row_src and a_lds
        for (int i = tid; i < MT; i += kThreads) {
            int src = -1;
            if (i < rows) src = FC1 ? p.sorted[row0 + i] / p.top_k : row0 + i;
            row_src[i] = src;
        }
        __syncthreads();

        uint32_t a_stage[kChunks][16];
        Span<BITS> sp[4];
        RawParams bp[4];
        auto load_step = [&](int s) {
            const int k0 = s * kSuperK;
#pragma unroll
            for (int j = 0; j < kChunks; ++j) {
                const int q = tid + kThreads * j;
                const int src = row_src[q >> 2];
                if (src >= 0) {
                    load_a_span(a_src + (int64_t)src * K, k0 + 32 * (q & 3), a_stage[j]);
                } else {
#pragma unroll
                    for (int i = 0; i < 16; ++i) a_stage[j][i] = 0u;
                }
            }
            if (active) {
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    sp[nb] = load_span<BITS>(wr[nb].codes, k0 + 32 * g);
                    bp[nb] = load_params<ZP>(wr[nb], k0 + 32 * g, p.block_size);
                }
            }
        };

        f32x4 acc[MB][4];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

        load_step(0);
        for (int s = 0; s < n_super; ++s) {
            uint32_t* buf = a_lds[s & 1];
#pragma unroll
            for (int j = 0; j < kChunks; ++j) {
                const int q = tid + kThreads * j;
                uint32_t perm[16];
                permute_span<O>(a_stage[j], perm);
                uint32_t* dst = buf + (q >> 2) * kPitch + 16 * (q & 3);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    *reinterpret_cast<u32x4*>(dst + 4 * v) =
                        u32x4{perm[4 * v], perm[4 * v + 1], perm[4 * v + 2], perm[4 * v + 3]};
                }
            }
            Span<BITS> cur[4];
            RawParams cbp[4];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                cur[nb] = sp[nb];
                cbp[nb] = bp[nb];
            }
            __syncthreads();
            if (s + 1 < n_super) load_step(s + 1);  // in flight during the MFMAs below

            if (active) {
                const int kk = s * kSuperK + 32 * g;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    u32x4 bf[4];
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb) {
                        const RawParams rq = (two_blocks && t >= 2)
                                                 ? load_params<ZP>(wr[nb], kk + 16, p.block_size)
                                                 : cbp[nb];
                        const BlockParams q = decode_params<DT, BITS, ZP>(rq, p.w.zp_fallback);
                        bf[nb] = dequant_zp<DT, BITS, ZP>(cur[nb], t, q);
                    }
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        if (mb * 16 < rows) {
                            const u32x4 af = *reinterpret_cast<const u32x4*>(
                                buf + (mb * 16 + c) * kPitch + 16 * g + 4 * t);
#pragma unroll
                            for (int nb = 0; nb < 4; ++nb) {
                                acc[mb][nb] = Dt<DT>::mfma(af, bf[nb], acc[mb][nb]);
                            }
                        }
                    }
                }
            }
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

template <bool FC1, int DT, int BITS>
hipError_t launch_zp(const ProjLaunch& p, hipStream_t s)
{
    const dim3 grid((unsigned)p.grid), block(kThreads);
    constexpr int MT = kPrefillMT;
    switch (zp_mode(p.w)) {
    case kZpConst: hipLaunchKernelGGL((prefill_kernel<DT, BITS, FC1, MT, kZpConst>), grid, block, 0, s, p); break;
    case kZpTensor: hipLaunchKernelGGL((prefill_kernel<DT, BITS, FC1, MT, kZpTensor>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((prefill_kernel<DT, BITS, FC1, MT, kZpGeneric>), grid, block, 0, s, p); break;
    }
    return hipGetLastError();
}

template <bool FC1, int DT>
hipError_t launch_dt(const ProjLaunch& p, hipStream_t s)
{
    switch (p.w.bits) {
    case 2: return launch_zp<FC1, DT, 2>(p, s);
    case 3: return launch_zp<FC1, DT, 3>(p, s);
    case 4: return launch_zp<FC1, DT, 4>(p, s);
    default: return hipErrorInvalidValue;
    }
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

// gemm_decode.hip -- grouped projection for few routed rows per expert.
//
// When the expanded row count R = T*top_k is small [PR 33569: the decode
// GEMV handles up to 80 expanded rows], each selected expert's weights are
// streamed from HBM once per 16 of its rows, so time is set by packed-weight
// bytes.  A workgroup takes one work-list item {expert, m, n}: up to 16 rows
// of the expert against NB column blocks of 16 weight rows.  Its four
// wavefronts split K (wavefront w takes super-steps w, w+4, ...); within a
// wavefront the 16 rows ride in the rows of a 16x16x32 MFMA, so the row count
// costs no VALU work and each weight element is dequantized once.
//
// Loads are ordered for latency.  The work-list item, the expert offsets and
// the item's 16 sorted route ids are uniform across the workgroup and come
// through scalar loads, which have their own counter, so they never hold up
// the vector loads.  Right after the item is known a wavefront issues the
// loads of a whole batch of super-steps (packed spans and the raw bits of
// block scales and zero points, none of which is consumed yet), then the A
// spans of its rows, and only then computes.  Each lane so keeps many loads
// in flight against HBM latency.  The four partial
// tiles are summed in LDS in a fixed order (no atomics), then the epilogue
// applies the gated activation (fc1) or writes float32 rows (fc2).
//
// RAW variant (block_size a multiple of 128, so every super-step lies in one
// quantization block): the B operand is the raw codes biased into exact dtype
// values (raw_step, one v_and_or_b32 per two weights) and the zero point and
// scale are applied per super-step in float32 from an extra MFMA against an
// all-ones B operand, which yields the row sums of A:
//   part = -(bias + zp) * rowsum + sum_t mfma(A_t, bias + codes_t)
//   acc += scale * part
// This halves the VALU work per weight, which is what bounds the kernel once
// all loads are in flight.
#include "gemm_common.h"

namespace qmoe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kBatch = 4;  // super-steps per wavefront whose loads are issued together

template <int DT, int BITS, bool FC1, int NB, int ZP, bool RAW>
__global__ __launch_bounds__(kThreads) void decode_kernel(ProjLaunch p,
                                                          const int32_t* __restrict__ wl,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ sorted,
                                                          const int32_t* __restrict__ n_items_ptr)
{
    static_assert(!FC1 || NB % 2 == 0, "fc1 column blocks come in gate/up pairs");
    constexpr Order O = RAW ? raw_order<BITS>() : code_order<DT, BITS>();
    constexpr int kCols = NB * 16;  // weight rows per item
    __shared__ float red[kWaves][kDecodeMT][kCols + 1];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int c = lane & 15;
    const int K = p.K;
    const int n_super = K / kSuperK;
    const int n_items = *n_items_ptr;
    const bool two_blocks = p.block_size < 32;  // a 32-code span crosses a block boundary
    const uint16_t* a_src = reinterpret_cast<const uint16_t*>(p.a);
    const uint32_t magic = opaque(DT == kF16 ? 0x64006400u : 0x43004300u);
    const u32x4 ones = {ones2<DT>(), ones2<DT>(), ones2<DT>(), ones2<DT>()};

    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int e = wl[3 * item + 0];
        const int mt = wl[3 * item + 1];
        const int nt = wl[3 * item + 2];

        int col0;
        WeightRow wr[NB];
        if constexpr (FC1) {
            col0 = nt * (kCols / 2);  // first activation column
#pragma unroll
            for (int q = 0; q < NB / 2; ++q) {
                const int64_t gate = (int64_t)e * p.N + 2 * (col0 + 16 * q + c);
                wr[2 * q] = weight_row(p.w, gate, K, p.block_size);
                wr[2 * q + 1] = weight_row(p.w, gate + 1, K, p.block_size);
            }
        } else {
            col0 = nt * kCols;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                wr[nb] = weight_row(p.w, (int64_t)e * p.N + col0 + 16 * nb + c, K, p.block_size);
            }
        }

        f32x4 acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

        int row0 = 0, rows = 0, src = -1;
        for (int s0 = wave; s0 < n_super; s0 += kWaves * kBatch) {
            Span<BITS> sp[kBatch][NB];
            RawParams rp[kBatch][NB];
            uint32_t araw[kBatch][16];
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int s = s0 + kWaves * b;
                if (s < n_super) {
                    const int kk = s * kSuperK + 32 * g;
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        sp[b][nb] = load_span<BITS>(wr[nb].codes, kk);
                        rp[b][nb] = load_params<ZP>(wr[nb], kk, p.block_size);
                    }
                }
            }
            if (s0 == wave) {
                // rows of the item and the A row of this lane (routed row c); the
                // 16 sorted ids are read as uniform scalars (the buffer has 16
                // entries of slack) and lane c picks its own
                row0 = offsets[e] + mt * kDecodeMT;
                rows = min(kDecodeMT, offsets[e + 1] - row0);
                int ids[kDecodeMT];
#pragma unroll
                for (int i = 0; i < kDecodeMT; ++i) ids[i] = sorted[row0 + i];
                int mine = ids[0];
#pragma unroll
                for (int i = 1; i < kDecodeMT; ++i) mine = c == i ? ids[i] : mine;
                src = c < rows ? (FC1 ? mine / p.top_k : row0 + c) : -1;
            }
            const uint16_t* a_row = a_src + (int64_t)(src >= 0 ? src : 0) * K;
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int s = s0 + kWaves * b;
                if (s < n_super) {
                    if (src >= 0) {
                        load_a_span(a_row, s * kSuperK + 32 * g, araw[b]);
                    } else {
#pragma unroll
                        for (int i = 0; i < 16; ++i) araw[b][i] = 0u;
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int s = s0 + kWaves * b;
                if (s < n_super) {
                    uint32_t af[16];
                    permute_span<O>(araw[b], af);
                    const int kk = s * kSuperK + 32 * g;
                    if constexpr (RAW) {
                        f32x4 rowsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const u32x4 a4 = {af[4 * t], af[4 * t + 1], af[4 * t + 2], af[4 * t + 3]};
                            rowsum = Dt<DT>::mfma(a4, ones, rowsum);
                        }
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) {
                            const BlockParams q = decode_params<DT, BITS, ZP>(rp[b][nb], p.w.zp_fallback);
                            f32x4 part = rowsum * (-(raw_bias<DT>() + q.zp));
#pragma unroll
                            for (int t = 0; t < 4; ++t) {
                                const u32x4 a4 = {af[4 * t], af[4 * t + 1], af[4 * t + 2], af[4 * t + 3]};
                                part = Dt<DT>::mfma(a4, raw_step<DT, BITS>(sp[b][nb], t, magic), part);
                            }
                            acc[nb] += part * q.scale;
                        }
                    } else {
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) {
                            const BlockParams q0 = decode_params<DT, BITS, ZP>(rp[b][nb], p.w.zp_fallback);
#pragma unroll
                            for (int t = 0; t < 4; ++t) {
                                BlockParams q = q0;
                                if (two_blocks && t >= 2) {
                                    q = decode_params<DT, BITS, ZP>(
                                        load_params<ZP>(wr[nb], kk + 16, p.block_size), p.w.zp_fallback);
                                }
                                const u32x4 a4 = {af[4 * t], af[4 * t + 1], af[4 * t + 2], af[4 * t + 3]};
                                const u32x4 bf = dequant_zp<DT, BITS, ZP>(sp[b][nb], t, q);
                                acc[nb] = Dt<DT>::mfma(a4, bf, acc[nb]);
                            }
                        }
                    }
                }
            }
        }

        if (n_super <= wave) {  // this wavefront had no super-step: still needs the rows
            row0 = offsets[e] + mt * kDecodeMT;
            rows = min(kDecodeMT, offsets[e + 1] - row0);
        }
        __syncthreads();  // the previous item is done reading red
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave][4 * g + i][nb * 16 + c] = acc[nb][i];
        __syncthreads();

        if constexpr (FC1) {
            const int I = p.N / 2;
            constexpr int kActCols = kCols / 2;
            for (int o = tid; o < kDecodeMT * kActCols; o += kThreads) {
                const int m = o / kActCols;
                const int j = o % kActCols;
                if (m >= rows) continue;
                const int gate_col = (j / 16) * 32 + (j % 16);  // blocks 2q gate, 2q+1 up
                float gate = 0.f, up = 0.f;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) {
                    gate += red[w][m][gate_col];
                    up += red[w][m][gate_col + 16];
                }
                uint16_t* out = reinterpret_cast<uint16_t*>(p.act_out) + (int64_t)(row0 + m) * I;
                out[col0 + j] = Dt<DT>::from_float(act_value<DT>(p.act, gate, up));
            }
        } else {
            for (int o = tid; o < kDecodeMT * kCols; o += kThreads) {
                const int m = o / kCols;
                const int h = o % kCols;
                if (m >= rows) continue;
                float v = 0.f;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) v += red[w][m][h];
                p.y2[(int64_t)sorted[row0 + m] * p.N + col0 + h] = v;
            }
        }
    }
}

template <bool FC1, int DT, int NB, int BITS, int ZP, bool RAW>
hipError_t launch_one(const ProjLaunch& p, hipStream_t s)
{
    hipLaunchKernelGGL((decode_kernel<DT, BITS, FC1, NB, ZP, RAW>), dim3((unsigned)p.grid),
                       dim3(kThreads), 0, s, p, p.worklist, p.offsets, p.sorted, p.n_items);
    return hipGetLastError();
}

template <bool FC1, int DT, int NB, int BITS>
hipError_t launch_zp(const ProjLaunch& p, hipStream_t s)
{
    const int zp = zp_mode(p.w);
    if (p.block_size % kSuperK == 0) {  // zero point applied in float32: any value works
        return zp == kZpTensor ? launch_one<FC1, DT, NB, BITS, kZpTensor, true>(p, s)
                               : launch_one<FC1, DT, NB, BITS, kZpConst, true>(p, s);
    }
    switch (zp) {
    case kZpConst: return launch_one<FC1, DT, NB, BITS, kZpConst, false>(p, s);
    case kZpTensor: return launch_one<FC1, DT, NB, BITS, kZpTensor, false>(p, s);
    default: return launch_one<FC1, DT, NB, BITS, kZpGeneric, false>(p, s);
    }
}

template <bool FC1, int DT, int NB>
hipError_t launch_dt(const ProjLaunch& p, hipStream_t s)
{
    switch (p.w.bits) {
    case 2: return launch_zp<FC1, DT, NB, 2>(p, s);
    case 3: return launch_zp<FC1, DT, NB, 3>(p, s);
    case 4: return launch_zp<FC1, DT, NB, 4>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_fc1_decode(const ProjLaunch& p, int dtype, hipStream_t s)
{
    return dtype == kBF16 ? launch_dt<true, kBF16, kDecodeFc1Blocks>(p, s)
                          : launch_dt<true, kF16, kDecodeFc1Blocks>(p, s);
}

hipError_t launch_fc2_decode(const ProjLaunch& p, int dtype, hipStream_t s)
{
    return dtype == kBF16 ? launch_dt<false, kBF16, kDecodeFc2Blocks>(p, s)
                          : launch_dt<false, kF16, kDecodeFc2Blocks>(p, s);
}

}  // namespace qmoe

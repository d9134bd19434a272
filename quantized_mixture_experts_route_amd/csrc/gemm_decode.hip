// gemm_decode.hip -- grouped projection for few routed rows per expert.
//
// When the expanded row count R = T*top_k is small [PR 33569: the decode
// GEMV handles up to 80 expanded rows], each selected expert's weights are
// streamed from HBM exactly once per 16 of its rows, so time is set by
// packed-weight bytes.  A workgroup takes one work-list item {expert, m, n}:
// up to 16 rows of the expert against 64 weight rows.  Its four wavefronts
// split K (wavefront w takes super-steps w, w+4, ...); within a wavefront the
// 16 rows ride in the rows of a 16x16x32 MFMA, so the row count costs no
// extra VALU work and only one dequantization per weight element is paid.
// The four partial 16x64 tiles are summed in LDS in a fixed order (no
// atomics), then the epilogue applies the gated activation (fc1) or writes
// float32 rows (fc2), as in the prefill kernel.
#include "gemm_common.h"

namespace qmoe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <int DT, int BITS, bool FC1>
__global__ __launch_bounds__(kThreads) void decode_kernel(ProjLaunch p)
{
    __shared__ float red[kWaves][kDecodeMT][kDecodeWeightRows + 1];

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
        const int row0 = p.offsets[e] + mt * kDecodeMT;
        const int rows = min(kDecodeMT, p.offsets[e + 1] - row0);

        int col0;
        int64_t wrow[4];
        if constexpr (FC1) {
            col0 = nt * kDecodeFc1Cols;
            wrow[0] = 2 * (col0 + c);
            wrow[1] = 2 * (col0 + c) + 1;
            wrow[2] = 2 * (col0 + 16 + c);
            wrow[3] = 2 * (col0 + 16 + c) + 1;
        } else {
            col0 = nt * kDecodeFc2Cols;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) wrow[nb] = col0 + nb * 16 + c;
        }
        WeightRow wr[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            wr[nb] = weight_row(p.w, (int64_t)e * p.N + wrow[nb], K, p.block_size);
        }
        // A operand row of this lane: routed row c of the item
        int src = -1;
        if (c < rows) src = FC1 ? p.sorted[row0 + c] / p.top_k : row0 + c;
        const uint16_t* a_row = a_src + (int64_t)(src >= 0 ? src : 0) * K;

        f32x4 acc[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int k0 = wave * kSuperK; k0 < K; k0 += kWaves * kSuperK) {
            Span<BITS> sp[4];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) sp[nb] = load_span<BITS>(wr[nb].codes, k0 + 32 * g);
            u32x4 af[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                af[t] = u32x4{0u, 0u, 0u, 0u};
                if (src >= 0) af[t] = *reinterpret_cast<const u32x4*>(a_row + k0 + 32 * g + 8 * t);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int kk = k0 + 32 * g + 8 * t;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    const u32x4 bf =
                        b_fragment<DT, BITS>(sp[nb], t, kk, wr[nb], p.w.zp_fallback, p.block_size);
                    acc[nb] = Dt<DT>::mfma(af[t], bf, acc[nb]);
                }
            }
        }

        __syncthreads();  // the previous item is done reading red
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave][4 * g + i][nb * 16 + c] = acc[nb][i];
        __syncthreads();

        if constexpr (FC1) {
            const int I = p.N / 2;
            for (int o = tid; o < kDecodeMT * kDecodeFc1Cols; o += kThreads) {
                const int m = o / kDecodeFc1Cols;
                const int j = o % kDecodeFc1Cols;
                if (m >= rows) continue;
                const int gate_col = (j / 16) * 32 + (j % 16);  // blocks 0/2 gate, 1/3 up
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
            for (int o = tid; o < kDecodeMT * kDecodeFc2Cols; o += kThreads) {
                const int m = o / kDecodeFc2Cols;
                const int h = o % kDecodeFc2Cols;
                if (m >= rows) continue;
                float v = 0.f;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) v += red[w][m][h];
                p.y2[(int64_t)p.sorted[row0 + m] * p.N + col0 + h] = v;
            }
        }
    }
}

template <bool FC1, int DT>
hipError_t launch_dt(const ProjLaunch& p, hipStream_t s)
{
    const dim3 grid((unsigned)p.grid), block(kThreads);
    switch (p.w.bits) {
    case 2: hipLaunchKernelGGL((decode_kernel<DT, 2, FC1>), grid, block, 0, s, p); break;
    case 3: hipLaunchKernelGGL((decode_kernel<DT, 3, FC1>), grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL((decode_kernel<DT, 4, FC1>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fc1_decode(const ProjLaunch& p, int dtype, hipStream_t s)
{
    return dtype == kBF16 ? launch_dt<true, kBF16>(p, s) : launch_dt<true, kF16>(p, s);
}

hipError_t launch_fc2_decode(const ProjLaunch& p, int dtype, hipStream_t s)
{
    return dtype == kBF16 ? launch_dt<false, kBF16>(p, s) : launch_dt<false, kF16>(p, s);
}

}  // namespace qmoe

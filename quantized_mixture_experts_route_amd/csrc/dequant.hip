// dequant.hip -- the projections' dequantization written out to memory, as a
// test hook.  It calls the same span load, group extraction, zero-point and
// dequant8 routines the projection kernels use, one thread per 32-code span.
#include "qmoe_device.h"
#include "qmoe_internal.h"

namespace qmoe {
namespace {

template <int DT, int BITS>
__global__ __launch_bounds__(256) void dequant_kernel(ProjArgs w, int64_t rows, int K,
                                                      int block_size, int32_t* codes_out,
                                                      uint16_t* w_out)
{
    const int spans = K / 32;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * spans) return;
    const int64_t row = idx / spans;
    const int k0 = (int)(idx % spans) * 32;
    const int n_blocks = K / block_size;
    const uint8_t* codes = w.codes + row * (int64_t)(K * BITS / 8);
    const uint16_t* scales = reinterpret_cast<const uint16_t*>(w.scales) + row * n_blocks;
    const uint8_t* zp = w.zp ? w.zp + row * zp_row_bytes(n_blocks, BITS) : nullptr;
    const Span<BITS> sp = load_span<BITS>(codes, k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int kk = k0 + 8 * i;
        const int blk = kk / block_size;
        const uint32_t group = span_group<BITS>(sp, i);
        const u32x4 v = dequant8<DT, BITS>(group, zero_point<BITS>(zp, blk, w.zp_fallback),
                                           Dt<DT>::to_float(scales[blk]));
        *reinterpret_cast<u32x4*>(w_out + row * K + kk) = v;
        if (codes_out) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                codes_out[row * K + kk + j] = (int32_t)((group >> (BITS * j)) & ((1u << BITS) - 1u));
            }
        }
    }
}

template <int DT>
hipError_t launch_dt(const ProjArgs& w, int64_t rows, int K, int block_size, int32_t* codes_out,
                     uint16_t* w_out, hipStream_t s)
{
    const int64_t n = rows * (K / 32);
    const dim3 grid((unsigned)((n + 255) / 256)), block(256);
    switch (w.bits) {
    case 2: hipLaunchKernelGGL((dequant_kernel<DT, 2>), grid, block, 0, s, w, rows, K, block_size, codes_out, w_out); break;
    case 3: hipLaunchKernelGGL((dequant_kernel<DT, 3>), grid, block, 0, s, w, rows, K, block_size, codes_out, w_out); break;
    case 4: hipLaunchKernelGGL((dequant_kernel<DT, 4>), grid, block, 0, s, w, rows, K, block_size, codes_out, w_out); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant(const ProjArgs& w, int64_t rows, int K, int block_size, int dtype,
                          int32_t* codes_out, void* w_out, hipStream_t s)
{
    uint16_t* o = reinterpret_cast<uint16_t*>(w_out);
    return dtype == kBF16 ? launch_dt<kBF16>(w, rows, K, block_size, codes_out, o, s)
                          : launch_dt<kF16>(w, rows, K, block_size, codes_out, o, s);
}

}  // namespace qmoe

// dequant.hip -- the projections' dequantization written out to memory, as a
// test hook.  One thread per 32-code span calls the same span load, zero-point
// and dequant_step / dequant_step_generic routines the projection kernels use,
// then stores every value at its input position (undoing the register order
// of code_order<DT, BITS>()).
#include "gemm_common.h"

namespace qmoe {
namespace {

template <int DT, int BITS, int ZP>
__global__ __launch_bounds__(256) void dequant_kernel(ProjArgs w, int64_t rows, int K,
                                                      int block_size, int32_t* codes_out,
                                                      uint16_t* w_out)
{
    constexpr Order O = code_order<DT, BITS>();
    const int spans = K / 32;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * spans) return;
    const int64_t row = idx / spans;
    const int k0 = (int)(idx % spans) * 32;
    const WeightRow r = weight_row(w, row, K, block_size);
    const Span<BITS> sp = load_span<BITS>(r.codes, k0);
    uint16_t* out = w_out + row * K + k0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        // steps 0-1 and 2-3 each lie within one block (block_size >= 16)
        const BlockParams q = decode_params<DT, BITS, ZP>(
            load_params<ZP>(r, k0 + 16 * (t >> 1), block_size), w.zp_fallback);
        const u32x4 v = dequant_zp<DT, BITS, ZP>(sp, t, q);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[order_lo(O, t, i)] = (uint16_t)(v[i] & 0xffffu);
            out[order_hi(O, t, i)] = (uint16_t)(v[i] >> 16);
        }
    }
    if (codes_out) {
#pragma unroll
        for (int j = 0; j < 32; ++j) codes_out[row * K + k0 + j] = (int32_t)span_code<BITS>(sp, j);
    }
}

template <int DT, int BITS>
hipError_t launch_zp(const ProjArgs& w, int64_t rows, int K, int block_size, int32_t* codes_out,
                     uint16_t* w_out, hipStream_t s)
{
    const int64_t n = rows * (K / 32);
    const dim3 grid((unsigned)((n + 255) / 256)), block(256);
    switch (zp_mode(w)) {
    case kZpConst: launch(dequant_kernel<DT, BITS, kZpConst>, grid, block, s, w, rows, K, block_size, codes_out, w_out); break;
    case kZpTensor: launch(dequant_kernel<DT, BITS, kZpTensor>, grid, block, s, w, rows, K, block_size, codes_out, w_out); break;
    default: launch(dequant_kernel<DT, BITS, kZpGeneric>, grid, block, s, w, rows, K, block_size, codes_out, w_out); break;
    }
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const ProjArgs& w, int64_t rows, int K, int block_size, int32_t* codes_out,
                     uint16_t* w_out, hipStream_t s)
{
    switch (w.bits) {
    case 2: return launch_zp<DT, 2>(w, rows, K, block_size, codes_out, w_out, s);
    case 3: return launch_zp<DT, 3>(w, rows, K, block_size, codes_out, w_out, s);
    case 4: return launch_zp<DT, 4>(w, rows, K, block_size, codes_out, w_out, s);
    default: return hipErrorInvalidValue;
    }
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

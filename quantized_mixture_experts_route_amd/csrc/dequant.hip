// dequant.hip -- the projections' unpacking and dequantization written out to
// memory, as test hooks.  One thread per 32-code span calls the same span
// load, zero-point and dequant_step / dequant_step_generic routines the
// prefill and row-block kernels use (dequant_kernel), or the raw-code
// routines of the decode kernels whose blocks span whole 128-input
// super-steps (raw_codes_kernel: raw_step with one base, raw_step_based with
// a base per register), then stores every value at its input position
// (undoing the register order of code_order / raw_order).
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

// The codes as the raw-code MFMA operands carry them: each 16-bit half is the
// dtype value base + code, exact, so subtracting the base in float32 gives the
// code back.  MULTI: raw_step_based with the streamed kernels' per-register
// bases (2- and 4-bit codes); otherwise raw_step with the single bias.
template <int DT, int BITS, bool MULTI>
__global__ __launch_bounds__(256) void raw_codes_kernel(const uint8_t* __restrict__ codes,
                                                        int64_t rows, int K,
                                                        int32_t* __restrict__ codes_out)
{
    constexpr Order O = raw_order<BITS>();
    const int spans = K / 32;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * spans) return;
    const int64_t row = idx / spans;
    const int k0 = (int)(idx % spans) * 32;
    const Span<BITS> sp = load_span<BITS>(codes + row * (int64_t)(K * BITS / 8), k0);
    uint32_t magic[4];
    float base[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if constexpr (MULTI) {
            magic[r] = opaque(raw_magic<DT, BITS>(r));
            base[r] = raw_base<DT, BITS>(r);
        } else {
            magic[r] = opaque(DT == kF16 ? 0x64006400u : 0x43004300u);
            base[r] = raw_bias<DT>();
        }
    }
    int32_t* out = codes_out + row * K + k0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        u32x4 v;
        if constexpr (MULTI) v = raw_step_based<DT, BITS>(sp, t, magic);
        else v = raw_step<DT, BITS>(sp, t, magic[0]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            out[order_lo(O, t, r)] = (int32_t)(Dt<DT>::to_float((uint16_t)(v[r] & 0xffffu)) - base[r]);
            out[order_hi(O, t, r)] = (int32_t)(Dt<DT>::to_float((uint16_t)(v[r] >> 16)) - base[r]);
        }
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
    case 1: return launch_zp<DT, 1>(w, rows, K, block_size, codes_out, w_out, s);
    case 2: return launch_zp<DT, 2>(w, rows, K, block_size, codes_out, w_out, s);
    case 3: return launch_zp<DT, 3>(w, rows, K, block_size, codes_out, w_out, s);
    case 4: return launch_zp<DT, 4>(w, rows, K, block_size, codes_out, w_out, s);
    case 8: return launch_zp<DT, 8>(w, rows, K, block_size, codes_out, w_out, s);
    default: return hipErrorInvalidValue;
    }
}

template <int DT, int BITS>
hipError_t launch_raw_bits(const uint8_t* codes, int64_t rows, int K, bool multi, int32_t* out,
                           hipStream_t s)
{
    const int64_t n = rows * (K / 32);
    const dim3 grid((unsigned)((n + 255) / 256)), block(256);
    if constexpr (BITS == 3) {
        if (multi) return hipErrorInvalidValue;  // the streamed kernels take 2- and 4-bit codes
        launch(raw_codes_kernel<DT, BITS, false>, grid, block, s, codes, rows, K, out);
    } else {
        if (multi) launch(raw_codes_kernel<DT, BITS, true>, grid, block, s, codes, rows, K, out);
        else launch(raw_codes_kernel<DT, BITS, false>, grid, block, s, codes, rows, K, out);
    }
    return hipGetLastError();
}

template <int DT>
hipError_t launch_raw_dt(const uint8_t* codes, int bits, int64_t rows, int K, bool multi,
                         int32_t* out, hipStream_t s)
{
    switch (bits) {
    case 2: return launch_raw_bits<DT, 2>(codes, rows, K, multi, out, s);
    case 3: return launch_raw_bits<DT, 3>(codes, rows, K, multi, out, s);
    case 4: return launch_raw_bits<DT, 4>(codes, rows, K, multi, out, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_raw_codes(const uint8_t* codes, int bits, int64_t rows, int K, int dtype,
                            bool multi, int32_t* codes_out, hipStream_t s)
{
    return dtype == kBF16 ? launch_raw_dt<kBF16>(codes, bits, rows, K, multi, codes_out, s)
                          : launch_raw_dt<kF16>(codes, bits, rows, K, multi, codes_out, s);
}

hipError_t launch_dequant(const ProjArgs& w, int64_t rows, int K, int block_size, int dtype,
                          int32_t* codes_out, void* w_out, hipStream_t s)
{
    uint16_t* o = reinterpret_cast<uint16_t*>(w_out);
    return dtype == kBF16 ? launch_dt<kBF16>(w, rows, K, block_size, codes_out, o, s)
                          : launch_dt<kF16>(w, rows, K, block_size, codes_out, o, s);
}

}  // namespace qmoe

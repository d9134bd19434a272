// qmoe_device.h -- device helpers shared by the gfx950 QMoE kernels:
// dtype traits, packed-code loads, the dequantization routine, gated
// activations and the MFMA operand types.
//
// Sources: [qmoe.rs] docs.rs onnx-runtime-ep-cuda src/kernels/qmoe.rs;
// [PR 32198] onnxruntime PR 32198 (int2 QMoE, GeGLU, fractional zero point);
// [PR 33569] onnxruntime PR 33569 (INT3 QMoE kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

constexpr int kWave = 64;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum : int { kF16 = 1, kBF16 = 2 };
enum : int { kSwiGLU = 0, kGeGLU = 1 };

// ---------------------------------------------------------------- dtypes
template <int DT>
struct Dt;

template <>
struct Dt<kF16> {
    __device__ static inline float to_float(uint16_t bits)
    {
        return (float)__builtin_bit_cast(_Float16, bits);
    }
    // Round to nearest even (the default rounding mode of v_cvt_f16_f32).
    __device__ static inline uint16_t from_float(float x)
    {
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    }
    __device__ static inline f32x4 mfma(u32x4 a, u32x4 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};

template <>
struct Dt<kBF16> {
    __device__ static inline float to_float(uint16_t bits)
    {
        return __builtin_bit_cast(float, (uint32_t)bits << 16);
    }
    // Round to nearest even on the float32 bit pattern (finite inputs; NaN
    // stays NaN by forcing a quiet mantissa bit).
    __device__ static inline uint16_t from_float(float x)
    {
        uint32_t u = __builtin_bit_cast(uint32_t, x);
        if ((u & 0x7fffffffu) > 0x7f800000u) {
            return (uint16_t)((u >> 16) | 0x40u);
        }
        u += 0x7fffu + ((u >> 16) & 1u);
        return (uint16_t)(u >> 16);
    }
    __device__ static inline f32x4 mfma(u32x4 a, u32x4 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

__device__ inline uint32_t pack2(uint16_t lo, uint16_t hi)
{
    return (uint32_t)lo | ((uint32_t)hi << 16);
}

// ---------------------------------------------------------------- codes
// A "span" is 32 consecutive codes of one weight row starting at a multiple
// of 32: 16 bytes at 4 bits, 8 bytes at 2 bits, 12 bytes at 3 bits.
// 2/4-bit codes fill each byte from the least significant bits up; 3-bit
// codes are 8 per little-endian 24-bit group [qmoe.rs decode_affine_weight;
// PR 33569, 24-bit 8-code INT3 unpacking].
template <int BITS>
struct Span {
    uint32_t w[BITS];
};

template <int BITS>
__device__ inline Span<BITS> load_span(const uint8_t* row, int k0)
{
    Span<BITS> s;
    const uint8_t* p = row + (size_t)k0 * BITS / 8;
    if constexpr (BITS == 4) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(p);
        s.w[0] = v.x; s.w[1] = v.y; s.w[2] = v.z; s.w[3] = v.w;
    } else if constexpr (BITS == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        s.w[0] = v.x; s.w[1] = v.y;
    } else {
        const uint3 v = *reinterpret_cast<const uint3*>(p);
        s.w[0] = v.x; s.w[1] = v.y; s.w[2] = v.z;
    }
    return s;
}

// Codes 8i..8i+7 of a span, code j at bits [BITS*j, BITS*j+BITS).
template <int BITS>
__device__ inline uint32_t span_group(const Span<BITS>& s, int i)
{
    if constexpr (BITS == 4) {
        return s.w[i];
    } else if constexpr (BITS == 2) {
        return (s.w[i >> 1] >> ((i & 1) * 16)) & 0xffffu;
    } else {
        // group i occupies bits [24i, 24i+24) of the 96-bit span; the
        // funnel shift (v_alignbit_b32) joins the two words it straddles.
        switch (i) {
        case 0: return s.w[0] & 0xffffffu;
        case 1: return __builtin_amdgcn_alignbit(s.w[1], s.w[0], 24) & 0xffffffu;
        case 2: return __builtin_amdgcn_alignbit(s.w[2], s.w[1], 16) & 0xffffffu;
        default: return s.w[2] >> 8;
        }
    }
}

// ---------------------------------------------------------------- zero points
// Zero-point tensor row bytes: 2/4-bit values packed like codes, 3-bit one byte each.
__host__ __device__ inline int zp_row_bytes(int n_blocks, int bits)
{
    return bits == 3 ? n_blocks : (n_blocks + (8 / bits) - 1) / (8 / bits);
}

// Zero point of quantization block `block` of a row: the tensor entry if the
// tensor is given, else `fallback` (the fractional offset, or 2^(bits-1))
// [qmoe.rs decode_affine_weight; PR 32198 zero_point_offset].
template <int BITS>
__device__ inline float zero_point(const uint8_t* zp_row, int block, float fallback)
{
    if (zp_row == nullptr) {
        return fallback;
    }
    if constexpr (BITS == 3) {
        return (float)zp_row[block];
    } else {
        constexpr int per = 8 / BITS;
        return (float)((zp_row[block / per] >> ((block % per) * BITS)) & ((1 << BITS) - 1));
    }
}

// ---------------------------------------------------------------- dequant
// Eight codes -> eight dtype values (code - zp) * scale, each rounded once to
// the dtype.  (code - zp) and its product with a 16-bit scale are exact in
// float32 for integer or half-integer zero points, so the result is the
// correctly rounded dequantized weight [PR 33569: dequantized weights are
// rounded to the activation type before accumulation].
template <int DT, int BITS>
__device__ inline u32x4 dequant8(uint32_t group, float zp, float scale)
{
    constexpr uint32_t mask = (1u << BITS) - 1u;
    uint16_t h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float q = (float)((group >> (BITS * j)) & mask);
        h[j] = Dt<DT>::from_float((q - zp) * scale);
    }
    return u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
}

// ---------------------------------------------------------------- activation
// Gated activations on an interleaved gate/up pair [qmoe.rs qmoe_activate
// (swiglu_value with alpha 1, beta 0, no limit; tanh-GELU constants);
// PR 32198 GeGLU].
template <int ACT>
__device__ inline float gated(float g, float u)
{
    if constexpr (ACT == kGeGLU) {
        const float inner = 0.7978845608028654f * (g + 0.044715f * g * g * g);
        return 0.5f * g * (1.0f + tanhf(inner)) * u;
    } else {
        // sigmoid computed without overflow for either sign of g
        const float e = expf(-fabsf(g));
        const float sig = g >= 0.0f ? 1.0f / (1.0f + e) : e / (1.0f + e);
        return g * sig * u;
    }
}

}  // namespace qmoe

namespace qmoe {

// ---------------------------------------------------------------- wave reductions
// Cross-lane exchange within 32-lane halves through ds_swizzle's bit-mask
// mode (lane i reads lane i ^ XOR); the two halves are then joined with
// readlane.  Every lane of the wave must be active.
template <int XOR>
__device__ inline uint32_t swizzle_xor(uint32_t v)
{
    static_assert(XOR > 0 && XOR < 32, "ds_swizzle bit-mask mode spans 32 lanes");
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1f | (XOR << 10));
}

__device__ inline uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int XOR>
__device__ inline uint64_t swizzle_xor_u64(uint64_t v)
{
    const uint32_t lo = swizzle_xor<XOR>((uint32_t)v);
    const uint32_t hi = swizzle_xor<XOR>((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

__device__ inline uint64_t readlane_u64(uint64_t v, int lane)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

// Wave-wide maximum of an unsigned 64-bit word, returned to every lane.
__device__ inline uint64_t wave_max_u64(uint64_t v)
{
    v = max_u64(v, swizzle_xor_u64<1>(v));
    v = max_u64(v, swizzle_xor_u64<2>(v));
    v = max_u64(v, swizzle_xor_u64<4>(v));
    v = max_u64(v, swizzle_xor_u64<8>(v));
    v = max_u64(v, swizzle_xor_u64<16>(v));
    return max_u64(readlane_u64(v, 0), readlane_u64(v, 32));
}

__device__ inline float swz_f32_max(float v, float o) { return o > v ? o : v; }

// Wave-wide maximum of NaN-free floats.
__device__ inline float wave_max_f32(float v)
{
#define QMOE_STEP(X) v = swz_f32_max(v, __builtin_bit_cast(float, swizzle_xor<X>(__builtin_bit_cast(uint32_t, v))))
    QMOE_STEP(1); QMOE_STEP(2); QMOE_STEP(4); QMOE_STEP(8); QMOE_STEP(16);
#undef QMOE_STEP
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    return swz_f32_max(a, b);
}

// Wave-wide float sum (butterfly order), returned to every lane.
__device__ inline float wave_sum_f32(float v)
{
#define QMOE_STEP(X) v += __builtin_bit_cast(float, swizzle_xor<X>(__builtin_bit_cast(uint32_t, v)))
    QMOE_STEP(1); QMOE_STEP(2); QMOE_STEP(4); QMOE_STEP(8); QMOE_STEP(16);
#undef QMOE_STEP
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    return a + b;
}

}  // namespace qmoe

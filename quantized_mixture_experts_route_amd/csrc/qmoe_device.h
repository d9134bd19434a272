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
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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
    } else if constexpr (BITS == 8) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(p);
        const u32x4 b = *reinterpret_cast<const u32x4*>(p + 16);
        s.w[0] = a.x; s.w[1] = a.y; s.w[2] = a.z; s.w[3] = a.w;
        s.w[4] = b.x; s.w[5] = b.y; s.w[6] = b.z; s.w[7] = b.w;
    } else if constexpr (BITS == 1) {
        s.w[0] = *reinterpret_cast<const uint32_t*>(p);
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

// ---------------------------------------------------------------- code order
// A 32-code span feeds four MFMA steps t = 0..3; each step takes 8 codes as
// four registers r of two 16-bit values.  A contraction is indifferent to
// which span codes go into which register as long as the A operand pairs the
// same inputs, so each (dtype, width) uses the order that unpacks cheapest:
//   kNatural : register (t, r) = codes (8t+2r, 8t+2r+1)
//   kStride4 : register (t, r) = codes (8t+r, 8t+r+4)       (pairs 16 bits apart
//              in a 4-bit word, 12 bits apart in a 24-bit int3 group)
//   kStride8 : register (t, r) = codes (16(t/2)+4(t%2)+r, ... + 8)  (pairs 16
//              bits apart in a 16-code int2 word)
enum class Order { kNatural, kStride4, kStride8 };

template <int DT, int BITS>
__host__ __device__ constexpr Order code_order()
{
    return BITS == 2 ? Order::kStride8 : Order::kStride4;
}

__host__ __device__ constexpr int order_lo(Order o, int t, int r)
{
    return o == Order::kNatural   ? 8 * t + 2 * r
           : o == Order::kStride4 ? 8 * t + r
                                  : 16 * (t >> 1) + 4 * (t & 1) + r;
}

__host__ __device__ constexpr int order_hi(Order o, int t, int r)
{
    return o == Order::kNatural   ? 8 * t + 2 * r + 1
           : o == Order::kStride4 ? 8 * t + r + 4
                                  : 16 * (t >> 1) + 4 * (t & 1) + r + 8;
}

// Code number c (0..31) of a span.
template <int BITS>
__device__ inline uint32_t span_code(const Span<BITS>& s, int c)
{
    if constexpr (BITS == 4) return (s.w[c >> 3] >> (4 * (c & 7))) & 15u;
    else if constexpr (BITS == 2) return (s.w[c >> 4] >> (2 * (c & 15))) & 3u;
    else if constexpr (BITS == 8) return (s.w[c >> 2] >> (8 * (c & 3))) & 255u;
    else if constexpr (BITS == 1) return (s.w[0] >> c) & 1u;
    else return (span_group<3>(s, c >> 3) >> (3 * (c & 7))) & 7u;
}

// 32 consecutive 16-bit A values (value 2i in the low half of in[i], 2i+1 in
// the high half) -> the A registers of the four steps in order O:
// out[4t+r] = (value order_lo(t,r), value order_hi(t,r)).
template <Order O>
__device__ inline void permute_span(const uint32_t (&in)[16], uint32_t (&out)[16])
{
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int lo = order_lo(O, t, r), hi = order_hi(O, t, r);
            if constexpr (O == Order::kNatural) {
                out[4 * t + r] = in[4 * t + r];
            } else {
                // v_perm_b32 picks bytes 0-3 from its second source, 4-7 from its first
                const uint32_t sel = ((lo & 1) ? 0x0302u : 0x0100u) |
                                     ((hi & 1) ? 0x07060000u : 0x05040000u);
                out[4 * t + r] = __builtin_amdgcn_perm(in[hi >> 1], in[lo >> 1], sel);
            }
        }
    }
}

// Chunk j of a super-step row (its 8 values 8j..8j+7, value 2i in the low
// half of in[i]) -> the A registers of MFMA step j % 4 of span j / 4, for the
// orders whose step reads one chunk (kNatural, kStride4).
template <Order O>
__device__ inline u32x4 permute_chunk(const u32x4& in)
{
    static_assert(O != Order::kStride8, "kStride8 steps read two chunks: use permute_chunk_pair");
    const uint32_t w[4] = {in.x, in.y, in.z, in.w};
    uint32_t out[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int lo = order_lo(O, 0, r), hi = order_hi(O, 0, r);
        if constexpr (O == Order::kNatural) {
            out[r] = w[r];
        } else {
            const uint32_t sel = ((lo & 1) ? 0x0302u : 0x0100u) |
                                 ((hi & 1) ? 0x07060000u : 0x05040000u);
            out[r] = __builtin_amdgcn_perm(w[hi >> 1], w[lo >> 1], sel);
        }
    }
    return u32x4{out[0], out[1], out[2], out[3]};
}

// kStride8: step 2m + u of a span reads values 4u..4u+3 of chunks 2m and
// 2m+1 (register r pairs value 4u+r of the first with value 4u+r of the
// second).  Lanes l and l^1 hold chunks 2m (even lane) and 2m+1 (odd lane) of
// one row; each keeps the half of its chunk that its own step reads, sends
// the other half to its neighbour, and returns the registers of step
// (its chunk) % 4.
__device__ inline u32x4 permute_chunk_pair(const u32x4& in, bool odd)
{
    const uint32_t send0 = odd ? in.x : in.z, send1 = odd ? in.y : in.w;
    const uint32_t keep0 = odd ? in.z : in.x, keep1 = odd ? in.w : in.y;
    constexpr int kSwapPairs = 0xb1;  // DPP quad_perm [1,0,3,2]
    const uint32_t recv0 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send0, kSwapPairs, 0xf, 0xf, false);
    const uint32_t recv1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send1, kSwapPairs, 0xf, 0xf, false);
    // v_perm_b32(a, b, sel): bytes 0-3 of b, 4-7 of a.  The even chunk's value
    // goes to the low half: the even lane's own (b), the odd lane's received (a).
    const uint32_t sel_lo = odd ? 0x01000504u : 0x05040100u;  // low 16 bits of both words
    const uint32_t sel_hi = odd ? 0x03020706u : 0x07060302u;  // high 16 bits of both words
    return u32x4{__builtin_amdgcn_perm(recv0, keep0, sel_lo), __builtin_amdgcn_perm(recv0, keep0, sel_hi),
                 __builtin_amdgcn_perm(recv1, keep1, sel_lo), __builtin_amdgcn_perm(recv1, keep1, sel_hi)};
}

// ---------------------------------------------------------------- dequant
// Zero points that are multiples of 1/2 and below 256 in magnitude (integer
// tensors, symmetric centres, the 1.5 offset of the int2 worked example) take
// the fast routines below; others take dequant_step_generic.
__host__ __device__ inline bool zp_is_half_integer(float zp)
{
    const float twice = zp * 2.0f;
    return twice == (float)(int)twice && zp > -256.0f && zp < 256.0f;
}

// Step t of a span -> four registers of dtype pairs in code_order<DT,BITS>,
// each value (code - zp) * scale rounded once to the dtype
// [PR 33569: dequantized weights are rounded to the activation type before
// accumulation].
//
// Both dtypes first place each code in the mantissa of an fp16 value: at
// bits 1.. of 0x6000 (512.0, spacing 0.5), so the register reads as the fp16
// pair (512 + code, 512 + code'); int4 with bf16 or an integer zero point
// uses two bases instead (1024 + code at bits 0..3, 64 + code at bits 4..7).
// fp16: subtracting base + zp is exact, and the packed multiply by the fp16
// scale rounds once.
// bf16: v_fma_mix_f32 forms (base + code)*s - (base + zp)*s from the fp16
// halves; both terms are exact in float32 (at most 11 + 8 significant bits),
// so the result is (code - zp)*s exactly and v_cvt_pk_bf16_f32 rounds once.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// A loop-invariant value the compiler must keep in a register (VGPR or
// SGPR) instead of folding it into a literal at every use.
__device__ inline uint32_t opaque(uint32_t v)
{
    asm volatile("" : "+v"(v));
    return v;
}

__device__ inline uint32_t opaque_s(uint32_t v)
{
    asm("" : "+s"(v));  // not volatile: identical masks may be shared and hoisted
    return v;
}

// (x & mask) | magic.  v_and_or_b32 has no literal-operand form on gfx950;
// with the mask in an SGPR and the magic in a VGPR the compiler selects the
// single instruction (and keeps track of its hazards itself).
__device__ inline uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic)
{
    return (x & opaque_s(mask)) | magic;
}

// INTZP: the zero point is known to be an integer (a uint8 tensor), which
// lets fp16 use the two-base int4 unpacking below too.
template <int DT, int BITS, bool INTZP = false>
__device__ inline u32x4 dequant_step(const Span<BITS>& sp, int t, float zp, float scale)
{
    // int4 with two bases: codes of nibbles 0/4 and 2/6 sit at mantissa bits
    // 0..3 of 1024.0 (spacing 1), nibbles 1/5 and 3/7 at bits 4..7 of 64.0
    // (spacing 1/16), so one shift serves four registers.  Exact for any
    // zero point in bf16 (applied in float32) and for integer ones in fp16.
    constexpr bool kTwoBase = BITS == 4 && (DT == kBF16 || INTZP);
    uint32_t raw[4];
    float base[2];  // base of even and odd registers
    if constexpr (kTwoBase) {
        const uint32_t lo = opaque(0x64006400u), hi = opaque(0x54005400u);
        const uint32_t g = sp.w[t];
        const uint32_t h = g >> 8;
        raw[0] = and_or(g, 0x000f000fu, lo);  // codes 0, 4
        raw[1] = and_or(g, 0x00f000f0u, hi);  // codes 1, 5
        raw[2] = and_or(h, 0x000f000fu, lo);  // codes 2, 6
        raw[3] = and_or(h, 0x00f000f0u, hi);  // codes 3, 7
        base[0] = 1024.0f;
        base[1] = 64.0f;
    } else {
        // codes to fp16 (512 + q): one v_and_or per register (two codes)
        const uint32_t kMagic = opaque(0x60006000u);
        base[0] = base[1] = 512.0f;
        if constexpr (BITS == 4) {
            const uint32_t g = sp.w[t];
            raw[0] = and_or(g << 1, 0x001e001eu, kMagic);
#pragma unroll
            for (int r = 1; r < 4; ++r) raw[r] = and_or(g >> (4 * r - 1), 0x001e001eu, kMagic);
        } else if constexpr (BITS == 2) {
            const uint32_t w = sp.w[t >> 1];
            const int j0 = 4 * (t & 1);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = j0 + r;
                raw[r] = and_or(j == 0 ? (w << 1) : (w >> (2 * j - 1)), 0x00060006u, kMagic);
            }
        } else if constexpr (BITS == 8) {
            // register r pairs bytes 8t + r and 8t + r + 4 (kStride4): one
            // v_perm_b32 places them at bits 0 and 16 with zero bytes beside them
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t sel = (uint32_t)r | 0x0c00u | ((uint32_t)(4 + r) << 16) | 0x0c000000u;
                const uint32_t y = __builtin_amdgcn_perm(sp.w[2 * t + 1], sp.w[2 * t], sel);
                raw[r] = and_or(y << 1, 0x01fe01feu, kMagic);
            }
        } else if constexpr (BITS == 1) {
            // register r pairs bits 8t + r and 8t + r + 4 of the span's word
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                // only bits 0 and 4 survive the mask, so the spread copies
                // (bit 0 to 1, bit 4 to 17) cannot collide with other codes
                const uint32_t x = (sp.w[0] >> (8 * t + r)) & 0x11u;
                raw[r] = and_or((x | (x << 12)) << 1, 0x00020002u, kMagic);
            }
        } else {
            const uint32_t g = span_group<3>(sp, t);
            const uint32_t y = (g & 0xfffu) | ((g << 4) & 0x0fff0000u);  // codes 4-7 to bit 16
            raw[0] = and_or(y << 1, 0x000e000eu, kMagic);
#pragma unroll
            for (int r = 1; r < 4; ++r) raw[r] = and_or(y >> (3 * r - 1), 0x000e000eu, kMagic);
        }
    }
    u32x4 out;
    if constexpr (DT == kF16) {
        // (base + q) - (base + zp) is exact in fp16 (half-integer zp at base
        // 512, integer zp at 1024 and 64); one rounding in the multiply
        const _Float16 sh = (_Float16)scale;
        const f16x2 s2 = {sh, sh};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const _Float16 c = (_Float16)(-(base[r & 1] + zp));
            const f16x2 c2 = {c, c};
            const f16x2 v = (__builtin_bit_cast(f16x2, raw[r]) + c2) * s2;
            out[r] = __builtin_bit_cast(uint32_t, v);
        }
    } else {
        // (base + q)*s - (base + zp)*s in one fused multiply-add with fp16
        // inputs (v_fma_mix_f32): both products are exact in float32, so the
        // result is (q - zp)*s exactly, rounded once to bf16
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const float c0 = -(base[0] + zp) * scale, c1 = -(base[1] + zp) * scale;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float c = (r & 1) ? c1 : c0;
            const f16x2 h = __builtin_bit_cast(f16x2, raw[r]);
            const bf16x2 v = {(__bf16)__builtin_fmaf((float)h.x, scale, c),
                              (__bf16)__builtin_fmaf((float)h.y, scale, c)};
            out[r] = __builtin_bit_cast(uint32_t, v);
        }
    }
    return out;
}

// ---------------------------------------------------------------- raw codes
// For blocks spanning whole 128-input super-steps the decode kernel feeds the
// MFMA the codes themselves, biased into exact dtype values: a code q placed
// at mantissa bit 0 of 0x6400 (fp16 1024.0) or 0x4300 (bf16 128.0) reads as
// kRawBias + q exactly.  The zero point and scale are applied afterwards in
// float32: sum_k (q_k - zp) x_k = sum_k (kRawBias + q_k) x_k - (kRawBias + zp) sum_k x_k.
// Both dtypes use the fp16 register orders here.
template <int BITS>
__host__ __device__ constexpr Order raw_order()
{
    return BITS == 2 ? Order::kStride8 : Order::kStride4;
}

template <int DT>
__host__ __device__ constexpr float raw_bias()
{
    return DT == kF16 ? 1024.0f : 128.0f;
}

// dtype 1.0 in both halves (MFMA B operand of all ones: row sums of A)
template <int DT>
__host__ __device__ constexpr uint32_t ones2()
{
    return DT == kF16 ? 0x3c003c00u : 0x3f803f80u;
}

// (x & mask) | (y & ~mask): v_bfi_b32 with the mask in an SGPR
__device__ inline uint32_t bfi(uint32_t mask, uint32_t x, uint32_t y)
{
    const uint32_t m = opaque_s(mask);
    return (x & m) | (y & ~m);
}

template <int DT, int BITS>
__device__ inline u32x4 raw_step(const Span<BITS>& sp, int t, uint32_t magic)
{
    u32x4 out;
    if constexpr (BITS == 4) {
        const uint32_t g = sp.w[t];
#pragma unroll
        for (int r = 0; r < 4; ++r) out[r] = and_or(r == 0 ? g : g >> (4 * r), 0x000f000fu, magic);
    } else if constexpr (BITS == 2) {
        const uint32_t w = sp.w[t >> 1];
        const int j0 = 4 * (t & 1);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = j0 + r;
            out[r] = and_or(j == 0 ? w : w >> (2 * j), 0x00030003u, magic);
        }
    } else {
        const uint32_t g = span_group<3>(sp, t);
        const uint32_t y = bfi(0xfffu, g, g << 4);  // codes 4-7 to bit 16 (bits 12-15 unused)
#pragma unroll
        for (int r = 0; r < 4; ++r) out[r] = and_or(r == 0 ? y : y >> (3 * r), 0x00070007u, magic);
    }
    return out;
}

// Multi-base raw codes (the streamed decode kernels): register r of an MFMA step takes its code pair from the packed
// word shifted right by raw_shift(r), at bits raw_pos(r) and raw_pos(r) + 16:
// int2 pairs sit 2r bits up (8 more on odd steps, taken out first), int4
// pairs 4(r & 1) bits up (8 more for r >= 2).  Fields must stay inside the
// mantissa (10 bits fp16, 7 bits bf16), so bf16 moves int2's fourth pair and
// int4's odd pairs down first.  The base is the power of two whose mantissa
// gives bit raw_pos(r) weight 1: 2^(m - raw_pos(r)).
template <int DT, int BITS>
__host__ __device__ constexpr int raw_shift(int r)
{
    if (BITS == 2) return (DT == kF16 || r < 3) ? 0 : 2;
    return (r < 2 ? 0 : 8) + ((DT == kBF16 && (r & 1)) ? 1 : 0);
}

template <int DT, int BITS>
__host__ __device__ constexpr int raw_pos(int r)
{
    if (BITS == 2) return (DT == kF16 || r < 3) ? 2 * r : 4;
    return (r & 1) ? (DT == kF16 ? 4 : 3) : 0;
}

template <int DT, int BITS>
__host__ __device__ constexpr float raw_base(int r)
{
    return (float)(1 << ((DT == kF16 ? 10 : 7) - raw_pos<DT, BITS>(r)));
}

template <int DT, int BITS>
__host__ __device__ constexpr uint32_t raw_magic(int r)
{
    // the dtype's bit pattern of raw_base(r), in both halves
    constexpr int kBias = DT == kF16 ? 15 : 127;
    constexpr int kMant = DT == kF16 ? 10 : 7;
    const uint32_t h = (uint32_t)(kBias + kMant - raw_pos<DT, BITS>(r)) << kMant;
    return h | (h << 16);
}

template <int DT, int BITS>
__device__ inline u32x4 raw_step_based(const Span<BITS>& sp, int t, const uint32_t (&magic)[4])
{
    constexpr uint32_t kField = BITS == 2 ? 0x00030003u : 0x000f000fu;
    const uint32_t x = BITS == 2 ? ((t & 1) ? sp.w[t >> 1] >> 8 : sp.w[t >> 1]) : sp.w[t];
    u32x4 out;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        out[r] = and_or(x >> raw_shift<DT, BITS>(r), kField << raw_pos<DT, BITS>(r), magic[r]);
    }
    return out;
}

// Any zero point: (code - zp) * scale in float32, rounded once to the dtype,
// in the same register order as dequant_step.
template <int DT, int BITS>
__device__ inline u32x4 dequant_step_generic(const Span<BITS>& sp, int t, float zp, float scale)
{
    constexpr Order O = code_order<DT, BITS>();
    u32x4 out;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float lo = ((float)span_code<BITS>(sp, order_lo(O, t, r)) - zp) * scale;
        const float hi = ((float)span_code<BITS>(sp, order_hi(O, t, r)) - zp) * scale;
        out[r] = pack2(Dt<DT>::from_float(lo), Dt<DT>::from_float(hi));
    }
    return out;
}

// ---------------------------------------------------------------- activation
// sigmoid(z) from e = exp(-|z|) in [0, 1], so that neither sign overflows:
// 1 / (1 + e) for z >= 0, e / (1 + e) below.  The exponential is the
// hardware base-2 one (v_exp_f32 of -|z| log2 e) and the quotient a hardware
// reciprocal (v_rcp_f32), each a few float32 ulps from the exact value; the
// activation is rounded to fp16/bf16 afterwards.  NaN stays NaN.
__device__ inline float sigmoid_fast(float z)
{
    const float e = __expf(-fabsf(z));
    return (z >= 0.0f ? 1.0f : e) * __builtin_amdgcn_rcpf(1.0f + e);
}

// Gated activations on an interleaved gate/up pair [qmoe.rs qmoe_activate
// (swiglu_value with alpha 1, beta 0, no limit; tanh-GELU constants);
// PR 32198 GeGLU].  tanh-GELU uses 0.5 (1 + tanh(x)) = sigmoid(2x).
template <int ACT>
__device__ inline float gated(float g, float u)
{
    if constexpr (ACT == kGeGLU) {
        const float inner = 0.7978845608028654f * (g + 0.044715f * g * g * g);
        return g * sigmoid_fast(2.0f * inner) * u;
    } else {
        return g * sigmoid_fast(g) * u;
    }
}

}  // namespace qmoe

namespace qmoe {

// ---------------------------------------------------------------- wave reductions
// Cross-lane exchange within 16-lane rows by DPP (a VALU operand modifier,
// no LDS round trip): lane i ^ 1 and lane i ^ 2 by quad permutes, then the
// 8-lane and 16-lane mirrors, which pair each lane with one of the other
// half once every quad (then every 8 lanes) holds its combined value.  The
// four rows are joined with readlane.  Every lane of the wave must be active.
enum : int { kDppXor1 = 0xb1, kDppXor2 = 0x4e, kDppHalfMirror = 0x141, kDppMirror = 0x140 };

template <int CTRL>
__device__ inline uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}

__device__ inline uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ inline uint64_t dpp_u64(uint64_t v)
{
    const uint32_t lo = dpp_u32<CTRL>((uint32_t)v);
    const uint32_t hi = dpp_u32<CTRL>((uint32_t)(v >> 32));
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
    v = max_u64(v, dpp_u64<kDppXor1>(v));
    v = max_u64(v, dpp_u64<kDppXor2>(v));
    v = max_u64(v, dpp_u64<kDppHalfMirror>(v));
    v = max_u64(v, dpp_u64<kDppMirror>(v));
    return max_u64(max_u64(readlane_u64(v, 0), readlane_u64(v, 16)),
                   max_u64(readlane_u64(v, 32), readlane_u64(v, 48)));
}

// Wave maximum of 32-bit unsigned values (same DPP steps as wave_max_u64).
__device__ inline uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, dpp_u32<kDppXor1>(v));
    v = max(v, dpp_u32<kDppXor2>(v));
    v = max(v, dpp_u32<kDppHalfMirror>(v));
    v = max(v, dpp_u32<kDppMirror>(v));
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(a, b), max(c, d));
}

// The same result as wave_max_u64 for words whose low halves differ between
// lanes (a key in the high half, a distinct index in the low half): the
// 32-bit maximum of the high halves, then the low half of the one lane that
// holds it; only when several lanes tie on the high half, a second 32-bit
// maximum over their low halves.  Two 32-bit reductions at most instead of
// one on 64-bit pairs.
__device__ inline uint64_t wave_max_keyed(uint64_t v)
{
    const uint32_t hi = (uint32_t)(v >> 32);
    const uint32_t top = wave_max_u32(hi);
    const uint64_t holders = __ballot(hi == top);
    uint32_t lo;
    if (__popcll(holders) == 1) {
        lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, (int)__builtin_ctzll(holders));
    } else {
        lo = wave_max_u32(hi == top ? (uint32_t)v : 0u);
    }
    return ((uint64_t)top << 32) | lo;
}

__device__ inline float f32_max(float v, float o) { return o > v ? o : v; }

template <int CTRL>
__device__ inline float dpp_f32(float v)
{
    return __builtin_bit_cast(float, dpp_u32<CTRL>(__builtin_bit_cast(uint32_t, v)));
}

__device__ inline float readlane_f32(float v, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Wave-wide maximum of NaN-free floats.
__device__ inline float wave_max_f32(float v)
{
    v = f32_max(v, dpp_f32<kDppXor1>(v));
    v = f32_max(v, dpp_f32<kDppXor2>(v));
    v = f32_max(v, dpp_f32<kDppHalfMirror>(v));
    v = f32_max(v, dpp_f32<kDppMirror>(v));
    return f32_max(f32_max(readlane_f32(v, 0), readlane_f32(v, 16)),
                   f32_max(readlane_f32(v, 32), readlane_f32(v, 48)));
}

// Wave-wide float sum (a fixed pairing order), returned to every lane.
__device__ inline float wave_sum_f32(float v)
{
    v += dpp_f32<kDppXor1>(v);
    v += dpp_f32<kDppXor2>(v);
    v += dpp_f32<kDppHalfMirror>(v);
    v += dpp_f32<kDppMirror>(v);
    return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
}

}  // namespace qmoe

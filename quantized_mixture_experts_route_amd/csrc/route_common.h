// route_common.h -- top-k selection of one token by one wavefront, shared by
// the stand-alone router and the fused decode plan.
//
// [qmoe.rs, total_order_key / route_value_is_better / qmoe_route]: experts
// are ranked by a total-order integer key of the float32 logit bits, equal
// keys going to the lower expert index; weights are exp(l - m) over the
// selected experts divided by their sum (normalize) or by the sum over all
// experts, m being the largest non-NaN logit.
//
// Each lane holds EPL experts (lane + 64 j) as 64-bit words (key in the high
// half, bitwise-inverted expert index in the low half), so one unsigned max
// picks the highest key and, among equal keys, the lowest index.  k rounds
// of a lane-local max plus a wave max (ds_swizzle + readlane) select the
// experts; the winner's word is cleared to 0, below any live word.
#pragma once

#include "qmoe_device.h"

namespace qmoe {

// Signed total-order key: negative floats get their magnitude bits flipped.
__device__ inline int32_t route_key(float v)
{
    const int32_t b = __builtin_bit_cast(int32_t, v);
    return b < 0 ? (b ^ 0x7fffffff) : b;
}

__device__ inline float key_to_logit(int32_t key)
{
    return __builtin_bit_cast(float, key < 0 ? (key ^ 0x7fffffff) : key);
}

// Routes one token; the whole wavefront calls it.  get(j) returns this lane's
// logit of expert lane + 64 j; it is called once for every j < EPL, also where
// lane + 64 j >= E (the value is then ignored), so that all of a lane's loads
// are issued before the first one is waited on.  For every slot s < top_k
// exactly one lane calls emit(s, expert, weight).  agg: NULL, or the token's
// row of aggregation weights [qmoe.rs, qmoe_route, its router_weights
// branch]: the logits then only select, and a selected expert's weight is
// agg[e], divided by the slot-order sum of the selected agg values when
// normalize is set (0 when that sum is 0).
template <int EPL, class Get, class Emit>
__device__ inline void route_values(int E, int top_k, int normalize, Get get, Emit emit,
                                    const float* agg = nullptr)
{
    const int lane = threadIdx.x & (kWave - 1);
    float val[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        val[j] = get(j);
    }
    uint64_t cand[EPL];
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const int e = lane + kWave * j;
        cand[j] = 0;
        if (e < E) {
            const float v = val[j];
            const uint32_t ukey = (uint32_t)route_key(v) ^ 0x80000000u;
            cand[j] = ((uint64_t)ukey << 32) | (uint32_t)~(uint32_t)e;
            if (v > m) {
                m = v;  // NaN compares false and is skipped
            }
        }
    }
    m = wave_max_f32(m);

    int32_t my_id[EPL];
    float my_num[EPL];
    float den = 0.0f;
    for (int s = 0; s < top_k; ++s) {
        uint64_t best = 0;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            best = max_u64(best, cand[j]);
        }
        best = wave_max_keyed(best);  // words are distinct: each holds its expert index
        const int e = (int)~(uint32_t)best;
        const float v = key_to_logit((int32_t)((uint32_t)(best >> 32) ^ 0x80000000u));
        const float num = agg ? agg[e] : expf(v - m);
        if (normalize) {
            den += num;  // slot order
        }
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            if (lane + kWave * j == e) {
                cand[j] = 0;
            }
            if (lane + kWave * j == s) {
                my_id[j] = e;
                my_num[j] = num;
            }
        }
    }
    if (agg && !normalize) {
        den = 1.0f;
    } else if (!normalize) {
        float part = 0.0f;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + kWave * j;
            if (e < E) {
                part += expf(val[j] - m);
            }
        }
        den = wave_sum_f32(part);
    }
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const int s = lane + kWave * j;
        if (s < top_k) {
            emit(s, my_id[j], (agg && den == 0.0f) ? 0.0f : my_num[j] / den);
        }
    }
}

// Routes the token whose E logits start at `row`.
template <int EPL, class Emit>
__device__ inline void route_token(const float* row, int E, int top_k, int normalize, Emit emit,
                                   const float* agg = nullptr)
{
    const int lane = threadIdx.x & (kWave - 1);
    route_values<EPL>(E, top_k, normalize, [&](int j) { return row[min(lane + kWave * j, E - 1)]; }, emit,
                      agg);
}

// Several tokens per wavefront: L lanes per token (L = 8 or 16, E <= L),
// lane L*i + j holding expert j of token i of the wavefront.  The same
// selection and arithmetic as route_values (the total-order key with the
// lowest index on ties, m the largest non-NaN logit, exp(l - m) summed in
// slot order), with every reduction confined to the token's L lanes by DPP
// (quad permutes, the 8-lane mirror, for L = 16 the 16-lane mirror); sums
// pair the lanes in the order route_values pairs them, and the lanes it adds
// beyond E hold zeros, so the weights are bit for bit route_values'.  No
// router_weights.  Lane L*i + s (s < top_k) calls emit(s, expert, weight);
// every lane must be active and `v` is ignored where j >= E.
template <int L, class Emit>
__device__ inline void route_group(int E, int top_k, int normalize, float v, Emit emit)
{
    static_assert(L == 8 || L == 16, "lanes per token");
    const int j = threadIdx.x & (L - 1);
    const bool ok = j < E;
    auto gmax64 = [](uint64_t x) {
        x = max_u64(x, dpp_u64<kDppXor1>(x));
        x = max_u64(x, dpp_u64<kDppXor2>(x));
        x = max_u64(x, dpp_u64<kDppHalfMirror>(x));
        if constexpr (L == 16) x = max_u64(x, dpp_u64<kDppMirror>(x));
        return x;
    };
    float m = (ok && v > -INFINITY) ? v : -INFINITY;  // NaN compares false and is skipped
    m = f32_max(m, dpp_f32<kDppXor1>(m));
    m = f32_max(m, dpp_f32<kDppXor2>(m));
    m = f32_max(m, dpp_f32<kDppHalfMirror>(m));
    if constexpr (L == 16) m = f32_max(m, dpp_f32<kDppMirror>(m));
    const uint32_t ukey = (uint32_t)route_key(v) ^ 0x80000000u;
    uint64_t cand = ok ? (((uint64_t)ukey << 32) | (uint32_t)~(uint32_t)j) : 0;
    int my_id = 0;
    float my_num = 0.0f, den = 0.0f;
    for (int s = 0; s < top_k; ++s) {
        const uint64_t best = gmax64(cand);  // words are distinct: each holds its expert index
        const int e = (int)~(uint32_t)best;
        const float bv = key_to_logit((int32_t)((uint32_t)(best >> 32) ^ 0x80000000u));
        const float num = expf(bv - m);
        if (normalize) den += num;  // slot order
        if (j == e) cand = 0;
        if (j == s) {
            my_id = e;
            my_num = num;
        }
    }
    if (!normalize) {
        float part = ok ? expf(v - m) : 0.0f;
        part += dpp_f32<kDppXor1>(part);
        part += dpp_f32<kDppXor2>(part);
        part += dpp_f32<kDppHalfMirror>(part);
        if constexpr (L == 16) part += dpp_f32<kDppMirror>(part);
        den = part;
    }
    if (j < top_k) emit(j, my_id, my_num / den);
}

}  // namespace qmoe

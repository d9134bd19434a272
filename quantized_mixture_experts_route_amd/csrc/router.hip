// router.hip -- router projection fused with top-k routing in one launch.
//
// [gemm_quant_moe.rs, moe_gate_topk_fused: a token's gate logits are its
// input row times the transposed gate weight matrix, followed by the top-k
// of those logits in the same kernel; moe.rs, the router GEMM that feeds the
// routing step.]  logits[t, e] = sum_h x[t, h] * w[e, h] with x and w in the
// layer's dtype, w row-major [E, H], products and sums in float32 on the
// v_mfma_f32_16x16x32_{f16,bf16} matrix cores; then each token's top-k and
// weights from those float32 logits, exactly as qmoe_route computes them
// (route_values: total-order key, lowest index on ties, exp(l - m) / D).
//
// A workgroup takes 16 tokens.  Lane 16g + c of an MFMA reads token c's row
// and expert c's gate row at the same 8 contraction positions (16 contiguous
// bytes each, so neither operand needs reordering), so each wave computes a
// 16-token x 16-expert logit block; blocks are dealt to the 8 wavefronts, and
// when the experts give fewer blocks than wavefronts (E <= 64) each block's K
// range is split between several wavefronts whose partial sums are added in
// a fixed order.  The logit tile stays in LDS, and each wavefront then routes
// tokens of the tile from it.
#include "qmoe_internal.h"
#include "route_common.h"

namespace qmoe {
namespace {

constexpr int kThreadsR = 512;
constexpr int kWavesR = kThreadsR / kWave;
constexpr int kTokR = 16;  // tokens per workgroup (MFMA rows)

template <int DT, int EPL>
__global__ __launch_bounds__(kThreadsR) void router_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ w,
                                                           int64_t T, int H, int E, int top_k,
                                                           int normalize,
                                                           float* __restrict__ logits_out,
                                                           int32_t* __restrict__ ids,
                                                           float* __restrict__ weights)
{
    constexpr int kPitch = EPL * kWave + 1;           // logit row pitch (floats)
    constexpr int kSplitMax = EPL == 1 ? kWavesR : 1;  // K parts of an expert block
    __shared__ float part[kSplitMax][kTokR][kPitch];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int c = lane & 15;
    const int64_t t0 = (int64_t)blockIdx.x * kTokR;
    const int n_eb = (E + 15) / 16;                 // 16-expert blocks (<= 4 when EPL == 1)
    const int split = EPL == 1 ? kWavesR / n_eb : 1;  // >= 2 when EPL == 1
    const int steps = H / 32;
    // rows past T or E repeat the last one: their results are never read
    const uint16_t* xa = x + min(t0 + c, T - 1) * (int64_t)H + 8 * g;

    for (int u = wave; u < n_eb * split; u += kWavesR) {
        const int eb = u / split;
        const int ks = u - eb * split;
        const int s_lo = steps * ks / split;
        const int s_hi = steps * (ks + 1) / split;
        const uint16_t* wb = w + (int64_t)min(eb * 16 + c, E - 1) * H + 8 * g;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int s = s_lo; s < s_hi; ++s) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(xa + 32 * s);
            const u32x4 b = *reinterpret_cast<const u32x4*>(wb + 32 * s);
            acc = Dt<DT>::mfma(a, b, acc);
        }
        // lane (g, c) holds tokens 4g..4g+3 of expert eb*16 + c
#pragma unroll
        for (int i = 0; i < 4; ++i) part[ks][4 * g + i][eb * 16 + c] = acc[i];
    }
    __syncthreads();

    for (int tt = wave; tt < kTokR; tt += kWavesR) {
        const int64_t t = t0 + tt;
        if (t >= T) break;  // uniform within the wavefront
        auto logit = [&](int e) {
            float v = part[0][tt][e];
            for (int ks = 1; ks < split; ++ks) v += part[ks][tt][e];  // K parts in order
            return v;
        };
        if (logits_out) {
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
                const int e = lane + kWave * j;
                if (e < E) logits_out[t * E + e] = logit(e);
            }
        }
        route_values<EPL>(E, top_k, normalize, [&](int j) { return logit(min(lane + kWave * j, E - 1)); },
                          [&](int s, int e, float wt) {
                              ids[t * top_k + s] = e;
                              weights[t * top_k + s] = wt;
                          });
    }
}

template <int DT, int EPL>
hipError_t run(const void* x, const void* w, int64_t T, int H, int E, int top_k, int normalize,
               float* logits_out, int32_t* ids, float* weights, hipStream_t s)
{
    const int64_t blocks = (T + kTokR - 1) / kTokR;
    launch(router_kernel<DT, EPL>, dim3((unsigned)blocks), dim3(kThreadsR), s,
           reinterpret_cast<const uint16_t*>(x), reinterpret_cast<const uint16_t*>(w), T, H, E,
           top_k, normalize, logits_out, ids, weights);
    return hipGetLastError();
}

template <int DT>
hipError_t run_dt(const void* x, const void* w, int64_t T, int H, int E, int top_k, int normalize,
                  float* logits_out, int32_t* ids, float* weights, hipStream_t s)
{
    const int epl = (E + kWave - 1) / kWave;
    if (epl <= 1) return run<DT, 1>(x, w, T, H, E, top_k, normalize, logits_out, ids, weights, s);
    if (epl <= 2) return run<DT, 2>(x, w, T, H, E, top_k, normalize, logits_out, ids, weights, s);
    if (epl <= 4) return run<DT, 4>(x, w, T, H, E, top_k, normalize, logits_out, ids, weights, s);
    if (epl <= 8) return run<DT, 8>(x, w, T, H, E, top_k, normalize, logits_out, ids, weights, s);
    return run<DT, 16>(x, w, T, H, E, top_k, normalize, logits_out, ids, weights, s);
}

}  // namespace

hipError_t launch_router(const void* hidden, const void* gate_weight, int64_t T, int H, int E,
                         int top_k, int normalize, int dtype, float* logits_out, int32_t* ids,
                         float* weights, hipStream_t s)
{
    if (E < 1 || E > 16 * kWave || H < 32 || H % 32) return hipErrorInvalidValue;
    return dtype == kBF16
               ? run_dt<kBF16>(hidden, gate_weight, T, H, E, top_k, normalize, logits_out, ids, weights, s)
               : run_dt<kF16>(hidden, gate_weight, T, H, E, top_k, normalize, logits_out, ids, weights, s);
}

}  // namespace qmoe

// shared.hip -- the shared-expert branch's token gate and gated add.
//
// [moe.rs: a shared gate GEMM gives one logit per token, and the token-gated
// add puts sigmoid(logit) times the shared expert's output onto the routed
// output.]  The shared expert's own projections run through the layer's
// grouped kernels as a one-expert layer (qmoe_forward_shared in
// qmoe_api.cpp); these two kernels are the parts around them:
//  - shared_gate_kernel: one wavefront per token forms sum_h x[t,h] g[h] in
//    float32 (16-byte loads, DPP wave sum) and stores sigmoid of it;
//  - gated_add_kernel: out[t,h] = RNE_dtype(out[t,h] + s[t] * shared[t,h]),
//    four values per thread.
#include "qmoe_device.h"
#include "qmoe_internal.h"

namespace qmoe {
namespace {

// sigmoid without overflow for either sign [qmoe.rs, stable_sigmoid]
__device__ inline float stable_sigmoid(float z)
{
    if (z >= 0.0f) return 1.0f / (1.0f + expf(-z));
    const float e = expf(z);
    return e / (1.0f + e);
}

template <int DT>
__global__ __launch_bounds__(256) void shared_gate_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ gate,
                                                          int64_t T, int H,
                                                          float* __restrict__ s_out)
{
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // whole wavefront
    const int lane = threadIdx.x & 63;
    const uint16_t* row = x + t * H;
    float acc = 0.0f;
    for (int h = 8 * lane; h < H; h += 8 * kWave) {  // H is a multiple of 8
        const u32x4 a = *reinterpret_cast<const u32x4*>(row + h);
        const u32x4 b = *reinterpret_cast<const u32x4*>(gate + h);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc += Dt<DT>::to_float((uint16_t)(a[i] & 0xffffu)) * Dt<DT>::to_float((uint16_t)(b[i] & 0xffffu));
            acc += Dt<DT>::to_float((uint16_t)(a[i] >> 16)) * Dt<DT>::to_float((uint16_t)(b[i] >> 16));
        }
    }
    acc = wave_sum_f32(acc);
    if (lane == 0) s_out[t] = stable_sigmoid(acc);
}

template <int DT>
__global__ __launch_bounds__(256) void gated_add_kernel(uint16_t* __restrict__ out,
                                                        const uint16_t* __restrict__ shared,
                                                        const float* __restrict__ s, int64_t T,
                                                        int H)
{
    const int64_t quads = H / 4;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= T * quads) return;
    const int64_t t = idx / quads;
    const int64_t off = t * H + (idx - t * quads) * 4;
    const float g = s[t];
    const uint2 o = *reinterpret_cast<const uint2*>(out + off);
    const uint2 v = *reinterpret_cast<const uint2*>(shared + off);
    auto one = [&](uint32_t ow, uint32_t vw, int half) {
        const uint16_t a = (uint16_t)(half ? ow >> 16 : ow & 0xffffu);
        const uint16_t b = (uint16_t)(half ? vw >> 16 : vw & 0xffffu);
        return Dt<DT>::from_float(Dt<DT>::to_float(a) + g * Dt<DT>::to_float(b));
    };
    uint2 r;
    r.x = pack2(one(o.x, v.x, 0), one(o.x, v.x, 1));
    r.y = pack2(one(o.y, v.y, 0), one(o.y, v.y, 1));
    *reinterpret_cast<uint2*>(out + off) = r;
}

}  // namespace

hipError_t launch_shared_gate(const void* hidden, const void* gate, int64_t T, int H, int dtype,
                              float* s_out, hipStream_t s)
{
    const dim3 grid((unsigned)((T + 3) / 4)), block(256);
    const uint16_t* x = reinterpret_cast<const uint16_t*>(hidden);
    const uint16_t* g = reinterpret_cast<const uint16_t*>(gate);
    if (dtype == kBF16) launch(shared_gate_kernel<kBF16>, grid, block, s, x, g, T, H, s_out);
    else launch(shared_gate_kernel<kF16>, grid, block, s, x, g, T, H, s_out);
    return hipGetLastError();
}

hipError_t launch_gated_add(void* out, const void* shared, const float* s_in, int64_t T, int H,
                            int dtype, hipStream_t s)
{
    const int64_t n = T * (H / 4);
    const dim3 grid((unsigned)((n + 255) / 256)), block(256);
    uint16_t* o = reinterpret_cast<uint16_t*>(out);
    const uint16_t* v = reinterpret_cast<const uint16_t*>(shared);
    if (dtype == kBF16) launch(gated_add_kernel<kBF16>, grid, block, s, o, v, s_in, T, H);
    else launch(gated_add_kernel<kF16>, grid, block, s, o, v, s_in, T, H);
    return hipGetLastError();
}

}  // namespace qmoe

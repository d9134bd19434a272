// combine.hip -- routing-weighted sum of the fc2 rows of each token.
//
// [qmoe.rs, qmoe_combine]: out[t, h] = sum over slots s = 0..k-1, in slot
// order, of w[t, s] * y2[t*k + s, h], accumulated in float32 and rounded once
// to the output dtype.  Each thread owns four consecutive h of one token, so
// there are no atomics and the result is deterministic.  When fc2 split its
// K range, each y2 row is first summed over its parts, in part order.
#include "qmoe_device.h"
#include "qmoe_internal.h"

namespace qmoe {
namespace {

// KMAX > 0: top_k <= KMAX, and every slot's rows (parts 0 and 1) are
// requested before any is added, so the loads overlap; the sums keep the
// order of the generic loop (KMAX = 0).
template <int DT, int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y2, int parts,
                                                      int64_t part_stride,
                                                      const float* __restrict__ w, int64_t T,
                                                      int H, int top_k,
                                                      uint16_t* __restrict__ out)
{
    const int64_t quads = (int64_t)H / 4;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= T * quads) return;
    const int64_t t = idx / quads;
    const int64_t h = (idx % quads) * 4;
    auto add = [](float4& v, const float4& u) {
        v.x += u.x;
        v.y += u.y;
        v.z += u.z;
        v.w += u.w;
    };
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (KMAX > 0) {
        float4 v[KMAX], u[KMAX];
        float wt[KMAX];
#pragma unroll
        for (int s = 0; s < KMAX; ++s) {
            if (s < top_k) {
                const int64_t r = t * top_k + s;
                wt[s] = w[r];
                v[s] = *reinterpret_cast<const float4*>(y2 + r * H + h);
                if (parts > 1) u[s] = *reinterpret_cast<const float4*>(y2 + part_stride + r * H + h);
            }
        }
#pragma unroll
        for (int s = 0; s < KMAX; ++s) {
            if (s < top_k) {
                const int64_t r = t * top_k + s;
                if (parts > 1) add(v[s], u[s]);
                for (int q = 2; q < parts; ++q) add(v[s], *reinterpret_cast<const float4*>(y2 + q * part_stride + r * H + h));
                sum.x += wt[s] * v[s].x;
                sum.y += wt[s] * v[s].y;
                sum.z += wt[s] * v[s].z;
                sum.w += wt[s] * v[s].w;
            }
        }
    } else {
        for (int s = 0; s < top_k; ++s) {
            const int64_t r = t * top_k + s;
            const float wt = w[r];
            float4 v = *reinterpret_cast<const float4*>(y2 + r * H + h);
            for (int q = 1; q < parts; ++q) add(v, *reinterpret_cast<const float4*>(y2 + q * part_stride + r * H + h));
            sum.x += wt * v.x;
            sum.y += wt * v.y;
            sum.z += wt * v.z;
            sum.w += wt * v.w;
        }
    }
    uint2 packed;
    packed.x = pack2(Dt<DT>::from_float(sum.x), Dt<DT>::from_float(sum.y));
    packed.y = pack2(Dt<DT>::from_float(sum.z), Dt<DT>::from_float(sum.w));
    *reinterpret_cast<uint2*>(out + t * H + h) = packed;
}

template <int DT>
void launch_dt(dim3 grid, dim3 block, hipStream_t s, const float* y2, int parts, int64_t part_stride,
               const float* weights, int64_t T, int H, int top_k, uint16_t* o)
{
    if (top_k <= 2) launch(combine_kernel<DT, 2>, grid, block, s, y2, parts, part_stride, weights, T, H, top_k, o);
    else if (top_k <= 4) launch(combine_kernel<DT, 4>, grid, block, s, y2, parts, part_stride, weights, T, H, top_k, o);
    else if (top_k <= 8) launch(combine_kernel<DT, 8>, grid, block, s, y2, parts, part_stride, weights, T, H, top_k, o);
    else if (top_k <= 16) launch(combine_kernel<DT, 16>, grid, block, s, y2, parts, part_stride, weights, T, H, top_k, o);
    else launch(combine_kernel<DT, 0>, grid, block, s, y2, parts, part_stride, weights, T, H, top_k, o);
}

}  // namespace

hipError_t launch_combine(const float* y2, int parts, int64_t part_stride, const float* weights,
                          int64_t T, int H, int top_k, void* out, int dtype, hipStream_t s)
{
    const int64_t n = T * (H / 4);
    const dim3 grid((unsigned)((n + 255) / 256)), block(256);
    uint16_t* o = reinterpret_cast<uint16_t*>(out);
    if (dtype == kBF16) launch_dt<kBF16>(grid, block, s, y2, parts, part_stride, weights, T, H, top_k, o);
    else launch_dt<kF16>(grid, block, s, y2, parts, part_stride, weights, T, H, top_k, o);
    return hipGetLastError();
}

}  // namespace qmoe

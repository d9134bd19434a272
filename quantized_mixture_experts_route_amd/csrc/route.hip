// route.hip -- top-k expert routing, one wavefront per token (route_token in
// route_common.h holds the selection and the weights).
#include "qmoe_internal.h"
#include "route_common.h"

namespace qmoe {
namespace {

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ agg, int64_t T,
                                                    int E, int top_k, int normalize,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ weights)
{
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) {
        return;  // whole wavefront leaves together
    }
    route_token<EPL>(logits + t * E, E, top_k, normalize, [&](int s, int e, float w) {
        ids[t * top_k + s] = e;
        weights[t * top_k + s] = w;
    }, agg ? agg + t * E : nullptr);
}

template <int EPL>
hipError_t launch_epl(const float* logits, const float* agg, int64_t T, int E, int top_k,
                     int normalize, int32_t* ids, float* weights, hipStream_t s)
{
    const int64_t blocks = (T + 3) / 4;
    launch(route_kernel<EPL>, dim3((unsigned)blocks), dim3(256), s, logits, agg, T, E,
                       top_k, normalize, ids, weights);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const float* logits, int64_t T, int E, int top_k, int normalize,
                        int32_t* ids, float* weights, hipStream_t s, const float* agg)
{
    const int epl = (E + kWave - 1) / kWave;
    if (epl <= 1) return launch_epl<1>(logits, agg, T, E, top_k, normalize, ids, weights, s);
    if (epl <= 2) return launch_epl<2>(logits, agg, T, E, top_k, normalize, ids, weights, s);
    if (epl <= 4) return launch_epl<4>(logits, agg, T, E, top_k, normalize, ids, weights, s);
    if (epl <= 8) return launch_epl<8>(logits, agg, T, E, top_k, normalize, ids, weights, s);
    return launch_epl<16>(logits, agg, T, E, top_k, normalize, ids, weights, s);
}

}  // namespace qmoe

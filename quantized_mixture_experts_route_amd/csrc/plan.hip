// plan.hip -- fused routing and grouping for the decode path (few routes).
//
// One workgroup does the whole plan of a decode layer call, so the two
// projections start after a single small launch:
//  1. routing, one wavefront per token (route_token: [qmoe.rs, qmoe_route]);
//  2. the stable grouping of routes by expert [qmoe.rs, launch_grouping]:
//     with R <= 128 routes held in LDS, route r's sorted position is the
//     number of routes with a smaller expert plus the number of earlier
//     routes with the same expert (a direct rank, no scan);
//  3. the m-tile list [gemm_quant_moe.rs, moe_build_tile_worklist, without
//     the n dimension]: every 16 consecutive sorted routes of one expert
//     form a tile, experts ascending.  A tile is kDecodeTileInts int32:
//     {expert, first sorted row, rows, 0, token ids[16], route ids[16]},
//     zero past `rows`.  Both projections enumerate (tile, n-block) items
//     from the same list, so it is written once.
// The expert offsets and sorted route array are not materialized: the tile
// carries the rows' token ids (fc1 A rows) and route ids (fc2 outputs).
#include "qmoe_internal.h"
#include "route_common.h"

namespace qmoe {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
static_assert(kDecodeMaxRoutes <= 2 * kWave, "ranks use two wavefronts");

template <int EPL>
__global__ __launch_bounds__(kThreads) void decode_plan_kernel(
    const float* __restrict__ logits, int T, int E, int top_k, int normalize,
    float* __restrict__ weights, int32_t* __restrict__ ids_out, float* __restrict__ w_out,
    int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles, int32_t* __restrict__ counters,
    int n_counters, const float* __restrict__ agg)
{
    __shared__ __attribute__((aligned(16))) int s_e[kDecodeMaxRoutes];  // expert of route r
    __shared__ int s_route[kDecodeMaxRoutes];  // route at sorted position p
    __shared__ int s_end[kDecodeMaxRoutes];    // end of position p's expert group
    __shared__ int s_tile_pos[kDecodeMaxRoutes];
    __shared__ int s_wave_starts[2];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & (kWave - 1);
    const int R = T * top_k;

    // routes past R keep a sentinel above every expert, so the rank loop
    // reads the whole table without a bound
    if (tid >= R && tid < kDecodeMaxRoutes) s_e[tid] = INT32_MAX;
    // the fc2 launch's column-block counters (combine folded into fc2) start at zero
    for (int i = tid; i < n_counters; i += kThreads) {
        __hip_atomic_store(&counters[i], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // 1) routing
    for (int t = wave; t < T; t += kWaves) {
        route_token<EPL>(logits + (int64_t)t * E, E, top_k, normalize, [&](int s, int e, float w) {
            const int r = t * top_k + s;
            s_e[r] = e;
            weights[r] = w;
            if (ids_out) ids_out[r] = e;
            if (w_out) w_out[r] = w;
        }, agg ? agg + (int64_t)t * E : nullptr);
    }
    __syncthreads();

    // 2) stable rank of every route by expert: four threads per route, each
    //    counting over a quarter of the table (16-byte reads, all issued at
    //    once), their counts summed across the four lanes
    {
        static_assert(kThreads == 4 * kDecodeMaxRoutes, "four threads per route");
        const int r = tid >> 2;
        const int quarter = tid & 3;
        const int e = s_e[r];
        int less = 0, before = 0, same = 0;
        const int4* tab = reinterpret_cast<const int4*>(s_e) + quarter * (kDecodeMaxRoutes / 16);
#pragma unroll
        for (int q4 = 0; q4 < kDecodeMaxRoutes / 16; ++q4) {
            const int4 f = tab[q4];
            const int fs[4] = {f.x, f.y, f.z, f.w};
            const int r0 = quarter * (kDecodeMaxRoutes / 4) + 4 * q4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                less += fs[i] < e;
                same += fs[i] == e;
                before += (fs[i] == e) & (r0 + i < r);
            }
        }
#pragma unroll
        for (int d = 1; d < 4; d <<= 1) {
            less += __shfl_xor(less, d, kWave);
            same += __shfl_xor(same, d, kWave);
            before += __shfl_xor(before, d, kWave);
        }
        if (quarter == 0 && r < R) {
            const int pos = less + before;
            s_route[pos] = r;
            s_end[pos] = less + same;
            // a tile starts every 16 rows of the expert's group
            s_tile_pos[pos] = (before % kDecodeMT) == 0 ? 1 : 0;
        }
    }
    __syncthreads();

    // 3) tile index of each tile start: starts at earlier positions
    const bool start = tid < R && s_tile_pos[tid] != 0;
    const uint64_t starts = __ballot(start);
    if (wave < 2 && lane == 0) s_wave_starts[wave] = __popcll(starts);
    __syncthreads();
    const int total = s_wave_starts[0] + (R > kWave ? s_wave_starts[1] : 0);
    const int rank = __popcll(starts & ((1ull << lane) - 1ull)) + (wave == 1 ? s_wave_starts[0] : 0);
    __syncthreads();  // every flag is read before positions overwrite it
    if (start) s_tile_pos[rank] = tid;
    __syncthreads();

    // one thread per (tile, row): the row's token and route ids, and rows 0..3
    // write the tile's header
    for (int u = tid; u < total * kDecodeMT; u += kThreads) {
        const int j = u / kDecodeMT;
        const int i = u - j * kDecodeMT;
        const int p0 = s_tile_pos[j];
        const int rows = min(kDecodeMT, s_end[p0] - p0);
        const int r = s_route[p0 + min(i, rows - 1)];
        int32_t* tile = tiles + (int64_t)j * kDecodeTileInts;
        tile[kDecodeTileTokens + i] = i < rows ? r / top_k : 0;
        tile[kDecodeTileRoutes + i] = i < rows ? r : 0;
        if (i < 4) tile[i] = i == 0 ? s_e[s_route[p0]] : i == 1 ? p0 : i == 2 ? rows : 0;
    }
    if (tid == 0) *n_tiles = total;
}

template <int EPL>
hipError_t launch_epl(const float* logits, int T, int E, int top_k, int normalize, float* weights,
                  int32_t* ids_out, float* w_out, int32_t* tiles, int32_t* n_tiles,
                  int32_t* counters, int n_counters, const float* agg, hipStream_t s)
{
    launch(decode_plan_kernel<EPL>, dim3(1), dim3(kThreads), s, logits, T, E, top_k,
                       normalize, weights, ids_out, w_out, tiles, n_tiles, counters, n_counters, agg);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_plan(const float* logits, int T, int E, int top_k, int normalize,
                              float* weights, int32_t* ids_out, float* w_out, int32_t* tiles,
                              int32_t* n_tiles, int32_t* counters, int n_counters, hipStream_t s,
                              const float* agg)
{
    if (T < 1 || T * top_k > kDecodeMaxRoutes) return hipErrorInvalidValue;
    const int epl = (E + kWave - 1) / kWave;
    if (epl <= 1) return launch_epl<1>(logits, T, E, top_k, normalize, weights, ids_out, w_out, tiles, n_tiles, counters, n_counters, agg, s);
    if (epl <= 2) return launch_epl<2>(logits, T, E, top_k, normalize, weights, ids_out, w_out, tiles, n_tiles, counters, n_counters, agg, s);
    if (epl <= 4) return launch_epl<4>(logits, T, E, top_k, normalize, weights, ids_out, w_out, tiles, n_tiles, counters, n_counters, agg, s);
    if (epl <= 8) return launch_epl<8>(logits, T, E, top_k, normalize, weights, ids_out, w_out, tiles, n_tiles, counters, n_counters, agg, s);
    return launch_epl<16>(logits, T, E, top_k, normalize, weights, ids_out, w_out, tiles, n_tiles, counters, n_counters, agg, s);
}

}  // namespace qmoe

// qmoe_internal.h -- host-side launch interface between the C ABI layer
// (qmoe_api.cpp) and the kernel translation units.  Not installed.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

// Kernel timer hook: when `start` is set, the next launch() records the pair
// in its own dispatch packet (the kernel's start and end, the timestamps a
// profiler reads) and clears it.  Thread-local; set by the C ABI's timer.
struct LaunchEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
LaunchEvents& launch_events();

// Sets the thread's qmoe_last_error() message ("qmoe: " + printf text) and
// returns `code`.
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

template <class Kernel, class... Args>
inline void launch(Kernel kernel, dim3 grid, dim3 block, hipStream_t s, Args... args)
{
    LaunchEvents& ev = launch_events();
    if (ev.start) {
        hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev.start, ev.stop, 0, args...);
        ev = LaunchEvents{};
    } else {
        hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
    }
}

// Tile shapes.  Prefill: a workgroup computes MT routed rows of one expert
// against 4*MT weight rows (MT/16 wavefronts x 64 rows); MT is
// kPrefillMTLarge or kPrefillMTSmall, chosen per layer call.  Decode: a workgroup computes up
// to 16 rows against kDecodeFc{1,2}Blocks column blocks of 16 weight rows,
// its 8 wavefronts splitting K.
constexpr int kPrefillMTLarge = 128;
constexpr int kPrefillMTSmall = 64;
constexpr int kDecodeMT = 16;
constexpr int kDecodeFc1Blocks = 4;  // 64 weight rows = 32 gate/up pairs
constexpr int kDecodeFc2Blocks = 2;  // 32 hidden columns
constexpr int kSuperK = 128;  // inputs per K super-step: 4 lane groups x 32 codes

// Output columns one work-list item covers (fc1 counts activation columns,
// i.e. gate/up row pairs; fc2 counts hidden columns): mt/16 wavefronts of
// nbw column blocks of 16 weight rows each.
constexpr int prefill_fc1_cols(int mt, int nbw = 4) { return mt / 2 * nbw; }
constexpr int prefill_fc2_cols(int mt, int nbw = 4) { return mt * nbw; }
constexpr int kDecodeFc1Cols = kDecodeFc1Blocks * 16 / 2;
constexpr int kDecodeFc2Cols = kDecodeFc2Blocks * 16;

// Decode m-tiles carry everything a workgroup needs in one scalar fetch:
// {expert, first sorted row, rows, 0, token ids[16], route ids[16]}, 0 past
// `rows`.  Item i of a decode projection with nt column blocks is tile
// i / nt, column block i % nt.
constexpr int kDecodeTileInts = 4 + 2 * kDecodeMT;
constexpr int kDecodeTileTokens = 4;               // first token id
constexpr int kDecodeTileRoutes = 4 + kDecodeMT;   // first route id
constexpr int kDecodeMaxRoutes = 128;  // routes the fused decode plan holds in LDS
constexpr int kDecodeRoutes = 80;      // decode path for R <= this (QMOE_DECODE_MAX_ROUTES)

struct ProjArgs {
    const uint8_t* codes;
    const void* scales;
    const uint8_t* zp;  // nullable
    float zp_fallback;  // fractional offset or symmetric centre
    int bits;
    int fast;           // every zero point is a multiple of 1/2 below 256: fast dequant
};

// The combine folded into a decode fc2 launch: every workgroup that writes
// fc2 rows of column block n arrives once on counters[n] (zeroed by the fc1 or
// plan launch before fc2 starts); the last to arrive sums, for the block's
// columns, each token's slots in slot order (the combine's arithmetic) and
// resets counters[n] to 0.  counters == nullptr: the separate combine runs.
struct FusedCombine {
    int32_t* counters;     // [column blocks of fc2]
    const float* weights;  // [T * top_k] routing weights
    void* out;             // dtype [T, H]
    int T;
};

// Gated-activation parameters (SwiGLU alpha, beta, limit).
struct ActParams {
    float alpha = 1.0f;
    float beta = 0.0f;
    float limit = __builtin_inff();
};

// One grouped projection over a work-list.
struct ProjLaunch {
    const void* a;            // fc1: hidden [T, K]; fc2: activations [R, K] in sorted order
    ProjArgs w;
    int K;                    // inputs
    int N;                    // weight rows (fc1: 2*I, fc2: H)
    int block_size;
    int top_k;
    int m_tile;               // prefill tile rows (kPrefillMTLarge or kPrefillMTSmall)
    int nbw = 4;              // prefill: MFMA column blocks per wavefront (2: the narrow 64-row tile)
    const int32_t* offsets;   // [E+1]
    const int32_t* sorted;    // [R]
    const int32_t* worklist;  // prefill: [cap, 3] triples; decode: m-tiles
    const int32_t* n_items;   // prefill: [1] items; decode: [1] m-tiles
    int64_t grid;             // decode: workgroups to launch; prefill: item bound
    int64_t tiles_cap;        // decode: capacity of the m-tile list
    int act;                  // fc1 only
    void* act_out;            // fc1: dtype [R, I] in sorted order
    float* y2;                // fc2: float32 [R, H] by route id (k_split parts)
    int k_split;              // prefill fc2: K parts (1, 2 or 4), each a work-list column block
    int64_t part_stride;      // prefill fc2: floats between the parts of y2
    FusedCombine fused;       // decode fc2: the combine folded in (counters nullable)
    // operator options (prefill and m-tile decode kernels only)
    ActParams ap;             // fc1: SwiGLU parameters
    int fusion = 1;           // fc1 gate/up layout: 1 interleaved, 2 halves, 0 separate fc3
    ProjArgs w3{};            // fc1 with fusion 0: the up projection [E, I, K]
    const float* bias = nullptr;   // nullable: fc1 [E, rows of fc1] / fc2 [E, N]
    const float* bias3 = nullptr;  // nullable: fc3 [E, I]
};

// Routing inputs and outputs of the expert-stationary decode kernels: fc1
// routes the tokens itself and writes the plan, fc2 reads offsets/sorted.
struct DecodePlan {
    const float* logits;  // [T, E]
    int T;
    int E;
    int normalize;
    float* weights;       // [R] routing weights (read by the combine)
    int32_t* ids_out;     // nullable [R]
    float* w_out;         // nullable [R]
    int32_t* offsets;     // [E+1] expert offsets into the sorted routes
    int32_t* sorted;      // [R] route ids grouped by expert, ascending
    int32_t* counters;    // nullable [n_counters]: zeroed by fc1's first workgroup
    int n_counters;
};

// agg: NULL or router_weights [T, E] (the weights of the selected experts)
hipError_t launch_route(const float* logits, int64_t T, int E, int top_k, int normalize,
                        int32_t* ids, float* weights, hipStream_t s, const float* agg = nullptr);

// Router projection + top-k (router.hip): logits = hidden @ gate_weight^T in
// float32 on the matrix cores, then route_values on them.
hipError_t launch_router(const void* hidden, const void* gate_weight, int64_t T, int H, int E,
                         int top_k, int normalize, int dtype, float* logits_out, int32_t* ids,
                         float* weights, hipStream_t s);

// Shared expert (shared.hip): s[t] = sigmoid(hidden[t] . gate) in float32,
// and out[t,h] = RNE(out[t,h] + s[t] * shared[t,h]) in the layer's dtype.
hipError_t launch_shared_gate(const void* hidden, const void* gate, int64_t T, int H, int dtype,
                              float* s_out, hipStream_t s);
hipError_t launch_gated_add(void* out, const void* shared, const float* s_in, int64_t T, int H,
                            int dtype, hipStream_t s);

hipError_t launch_group(const int32_t* ids, int R, int E, int m_tile, int nt1, int32_t* offsets,
                        int32_t* sorted, int32_t* wl1, int64_t cap1, int32_t* n1, int nt2,
                        int32_t* wl2, int64_t cap2, int32_t* n2, hipStream_t s);

// Routing plus the decode m-tile list in one workgroup (T*top_k <=
// kDecodeMaxRoutes).  ids_out / w_out may be NULL.
hipError_t launch_decode_plan(const float* logits, int T, int E, int top_k, int normalize,
                              float* weights, int32_t* ids_out, float* w_out, int32_t* tiles,
                              int32_t* n_tiles, int32_t* counters, int n_counters, hipStream_t s,
                              const float* agg = nullptr);

hipError_t launch_fc1_prefill(const ProjLaunch& p, int dtype, hipStream_t s);
hipError_t launch_fc2_prefill(const ProjLaunch& p, int dtype, hipStream_t s);
// plan == nullptr: the m-tile list path (p.worklist / p.n_items); otherwise
// the expert-stationary kernels (K <= 2048, E <= 64, R <= kDecodeMaxRoutes).
hipError_t launch_fc1_decode(const ProjLaunch& p, const DecodePlan* plan, int dtype, hipStream_t s);
hipError_t launch_fc2_decode(const ProjLaunch& p, const DecodePlan* plan, int dtype, hipStream_t s);

// Row-block decode projections over the m-tile list (tiles of at most
// max_rows <= 16 rows; a constant zero point, K <= 2048, 128 weight rows per
// workgroup).  rows_fits: the projection's shapes and scales suit the kernel.
bool rows_fits(const ProjArgs& w, int K, int N, int block_size);
hipError_t launch_rows_decode(const ProjLaunch& p, bool fc1, int max_rows, int dtype, hipStream_t s);

// Streamed decode projections (T <= 16, R = T*top_k <= 64, E <= 64): every expert's
// weights requested at launch and consumed piece by piece as they land; fc1
// routes the tokens itself and writes the plan.  stream_fits: the projection's
// shapes, widths and scales suit the kernel.
bool stream_fits(const ProjArgs& w, int K, int N, int block_size, bool fc1);
hipError_t launch_fc1_stream(const ProjLaunch& p, const DecodePlan& plan, int dtype, hipStream_t s);
hipError_t launch_fc2_stream(const ProjLaunch& p, const DecodePlan& plan, int dtype, hipStream_t s);

// y2 holds `parts` partial sums of the fc2 rows, part_stride floats apart;
// they are added in part order before the routing weights apply.
hipError_t launch_combine(const float* y2, int parts, int64_t part_stride, const float* weights,
                          int64_t T, int H, int top_k, void* out, int dtype, hipStream_t s);

hipError_t launch_dequant(const ProjArgs& w, int64_t rows, int K, int block_size, int dtype,
                          int32_t* codes_out, void* w_out, hipStream_t s);

// The codes as the decode kernels' raw-code MFMA operands carry them
// (multi: the streamed kernels' per-register bases, 2/4-bit only).
hipError_t launch_raw_codes(const uint8_t* codes, int bits, int64_t rows, int K, int dtype,
                            bool multi, int32_t* codes_out, hipStream_t s);

}  // namespace qmoe

// stubs.cpp -- host-only stand-ins for the kernel launchers and the few HIP
// runtime calls of qmoe_api.cpp, so that the library's host code (argument
// checks, workspace layout, path selection, dispatch) runs under AddressSanitizer
// and UndefinedBehaviorSanitizer on a machine without a GPU.
//
// Every launcher appends its name to a call log and checks that the buffers
// it was handed lie inside the workspace the driver registered; nothing is
// dereferenced, since the pointers stand for device memory.
#include "stubs.h"

#include <cstdio>
#include <cstdlib>

namespace stub {

std::vector<std::string> calls;
const char* ws_lo = nullptr;
const char* ws_hi = nullptr;
bool rows_ok = false;
bool stream_ok = false;
int events = 0;

void in_ws(const void* p, const char* what)
{
    if (!ws_lo || !p) return;
    const char* c = static_cast<const char*>(p);
    if (c < ws_lo || c >= ws_hi) {
        std::fprintf(stderr, "launcher got %s outside the workspace\n", what);
        std::abort();
    }
}

}  // namespace stub

namespace {

hipError_t log(const char* name)
{
    stub::calls.emplace_back(name);
    return hipSuccess;
}

void proj_ws(const qmoe::ProjLaunch& p)
{
    stub::in_ws(p.offsets, "offsets");
    stub::in_ws(p.sorted, "sorted");
    stub::in_ws(p.worklist, "worklist");
    stub::in_ws(p.n_items, "n_items");
    stub::in_ws(p.act_out, "act");
    stub::in_ws(p.y2, "y2");
}

}  // namespace

namespace qmoe {

hipError_t launch_route(const float*, int64_t, int, int, int, int32_t* ids, float* w, hipStream_t,
                        const float*)
{
    stub::in_ws(ids, "route ids");
    stub::in_ws(w, "route weights");
    return log("route");
}

hipError_t launch_router(const void*, const void*, int64_t, int, int, int, int, int, float*, int32_t*,
                         float*, hipStream_t)
{
    return log("router");
}

hipError_t launch_shared_gate(const void*, const void*, int64_t, int, int, float* s_out, hipStream_t)
{
    stub::in_ws(s_out, "shared gate");
    return log("shared_gate");
}

hipError_t launch_gated_add(void*, const void* shared, const float* s_in, int64_t, int, int, hipStream_t)
{
    stub::in_ws(shared, "shared output");
    stub::in_ws(s_in, "shared gate");
    return log("gated_add");
}

hipError_t launch_group(const int32_t*, int, int, int, int, int32_t* offsets, int32_t* sorted,
                        int32_t* wl1, int64_t, int32_t* n1, int, int32_t* wl2, int64_t, int32_t* n2,
                        hipStream_t)
{
    stub::in_ws(offsets, "offsets");
    stub::in_ws(sorted, "sorted");
    stub::in_ws(wl1, "wl1");
    stub::in_ws(n1, "n1");
    stub::in_ws(wl2, "wl2");
    stub::in_ws(n2, "n2");
    return log("group");
}

hipError_t launch_decode_plan(const float*, int, int, int, int, float* weights, int32_t*, float*,
                              int32_t* tiles, int32_t* n_tiles, int32_t* counters, int, hipStream_t,
                              const float*)
{
    stub::in_ws(weights, "plan weights");
    stub::in_ws(tiles, "tiles");
    stub::in_ws(n_tiles, "n_tiles");
    stub::in_ws(counters, "counters");
    return log("plan");
}

hipError_t launch_fc1_prefill(const ProjLaunch& p, int, hipStream_t)
{
    proj_ws(p);
    return log("fc1_prefill");
}

hipError_t launch_fc2_prefill(const ProjLaunch& p, int, hipStream_t)
{
    proj_ws(p);
    return log("fc2_prefill");
}

hipError_t launch_fc1_decode(const ProjLaunch& p, const DecodePlan*, int, hipStream_t)
{
    proj_ws(p);
    return log("fc1_decode");
}

hipError_t launch_fc2_decode(const ProjLaunch& p, const DecodePlan*, int, hipStream_t)
{
    proj_ws(p);
    return log("fc2_decode");
}

bool rows_fits(const ProjArgs&, int, int, int) { return stub::rows_ok; }

hipError_t launch_rows_decode(const ProjLaunch& p, bool fc1, int, int, hipStream_t)
{
    proj_ws(p);
    return log(fc1 ? "fc1_rows" : "fc2_rows");
}

bool stream_fits(const ProjArgs&, int, int, int, bool) { return stub::stream_ok; }

hipError_t launch_fc1_stream(const ProjLaunch& p, const DecodePlan& plan, int, hipStream_t)
{
    proj_ws(p);
    stub::in_ws(plan.offsets, "plan offsets");
    stub::in_ws(plan.sorted, "plan sorted");
    stub::in_ws(plan.weights, "plan weights");
    return log("fc1_stream");
}

hipError_t launch_fc2_stream(const ProjLaunch& p, const DecodePlan&, int, hipStream_t)
{
    proj_ws(p);
    stub::in_ws(p.fused.counters, "combine counters");
    return log("fc2_stream");
}

hipError_t launch_combine(const float* y2, int, int64_t, const float* weights, int64_t, int, int, void*,
                          int, hipStream_t)
{
    stub::in_ws(y2, "combine y2");
    stub::in_ws(weights, "combine weights");
    return log("combine");
}

hipError_t launch_dequant(const ProjArgs&, int64_t, int, int, int, int32_t*, void*, hipStream_t)
{
    return log("dequant");
}

hipError_t launch_raw_codes(const uint8_t*, int, int64_t, int, int, bool, int32_t*, hipStream_t)
{
    return log("raw_codes");
}

}  // namespace qmoe

// HIP runtime calls made by the host code itself
extern "C" {

hipError_t hipEventCreate(hipEvent_t* event)
{
    ++stub::events;
    *event = reinterpret_cast<hipEvent_t>(static_cast<uintptr_t>(0x1000 + 16 * stub::events));
    return hipSuccess;
}

hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }

hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t)
{
    *ms = 0.25f;
    return hipSuccess;
}

hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t)
{
    stub::calls.emplace_back("memcpy");
    return hipSuccess;
}

const char* hipGetErrorString(hipError_t) { return "stub error"; }

}  // extern "C"

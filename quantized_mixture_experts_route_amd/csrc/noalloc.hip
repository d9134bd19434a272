// noalloc.hip -- qmoe_forward_noalloc: the whole layer with its workspace in a
// fixed device array of this library instead of a caller buffer, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The array lives in the library's code object: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  Host code
// never passes the array's name to a kernel (on the host that name is a
// stand-in, not a device address): the first call on a device, with that
// device current, looks the device address up once with hipGetSymbolAddress
// and keeps it for that device; every later call passes that address as the
// workspace of qmoe_forward, whose kernels take it as an argument.  Nothing
// here calls hipMalloc, hipFree or any allocating routine.
//
// The forward path needs no zeroed workspace (every word it reads was
// written earlier in the same call), so nothing is cleared between calls.
// Calls that overlap in time on one GPU share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "qmoe.h"
#include "qmoe_internal.h"

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[QMOE_NOALLOC_SCRATCH_BYTES];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on the first call on
// that device), or nullptr with *err set.
void* device_scratch(hipError_t* err)
{
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        void* ptr = nullptr;
        *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        g_scratch[dev] = ptr;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" int qmoe_forward_noalloc(const void* hidden, const float* logits, int64_t T, int32_t H,
                                    int32_t I, int32_t E, const qmoe_proj* fc1,
                                    const qmoe_proj* fc2, float zero_point_offset,
                                    int32_t block_size, int32_t top_k, int32_t normalize,
                                    int32_t activation, int32_t dtype, void* out,
                                    int32_t* topk_ids_out, float* topk_w_out, void* stream)
{
    const size_t need = qmoe_workspace_size(T, H, I, E, top_k, dtype);
    if (need > (size_t)QMOE_NOALLOC_SCRATCH_BYTES) {
        return qmoe::set_error(QMOE_ERR_WORKSPACE,
                               "qmoe_forward_noalloc: these sizes need %zu bytes of workspace, "
                               "its fixed scratch holds %zu; call qmoe_forward with a workspace",
                               need, (size_t)QMOE_NOALLOC_SCRATCH_BYTES);
    }
    void* ws = nullptr;
    if (need > 0 && T > 0) {  // sizes qmoe_forward accepts and work to do
        hipError_t e;
        ws = device_scratch(&e);
        if (ws == nullptr) {
            return qmoe::set_error(QMOE_ERR_HIP, "qmoe_forward_noalloc: scratch address: %s",
                                   hipGetErrorString(e));
        }
    }
    // invalid sizes and T = 0 get qmoe_forward's own checks and messages (it
    // returns for T = 0, and rejects invalid sizes, before it reads the
    // workspace pointer)
    return qmoe_forward(hidden, logits, T, H, I, E, fc1, fc2, zero_point_offset, block_size, top_k,
                        normalize, activation, dtype, out, topk_ids_out, topk_w_out, ws,
                        (size_t)QMOE_NOALLOC_SCRATCH_BYTES, stream);
}

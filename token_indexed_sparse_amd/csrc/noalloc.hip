// qsa_forward_noalloc: the forward with its workspace in a fixed device array
// of the library instead of caller memory, for callers that cannot allocate.
//
// `scratch` below is a file-scope device array. In host code its name is a
// host-side stand-in, not a device address, so host code never passes it to a
// kernel or a copy: the first call on each device (with that device current)
// looks up the array's device address with hipGetSymbolAddress and keeps it
// per device, and every call passes that address as the forward's workspace.
// Each device holds its own copy of the array, at its own address, from then
// until the process ends. The forward clears on the device everything it
// needs cleared, so the contents a previous call left behind do not matter;
// calls that overlap on one device share the array and race.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "../../include/qsa.h"

namespace {

constexpr size_t kScratchBytes = QSA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_scratch[kMaxDevices];

// The device address of this device's array, or null if it cannot be had.
void *device_scratch()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(g_once[dev], [dev]() {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess) g_scratch[dev] = ptr;
    });
    return g_scratch[dev];
}

}  // namespace

extern "C" qsa_status qsa_forward_noalloc(const qsa_dims *dims, const void *q, const void *k,
                                          const void *v, const void *routes, float scale,
                                          void *out, float *out_fp32, float *lse, void *stream)
{
    // Validation that needs no device, before the address lookup: an invalid
    // call returns the status qsa_forward gives it (its workspace check comes
    // after every shape, pointer and scale check).
    const size_t need = qsa_forward_workspace_bytes(dims);
    if (need == 0 || !q || !k || !v || !routes || !out || !out_fp32 || !lse ||
        !(std::isfinite(scale) && scale > 0.f))
        return qsa_forward(dims, q, k, v, routes, scale, out, out_fp32, lse, nullptr, 0, stream);
    if (need > kScratchBytes) return QSA_ERR_SCRATCH;
    void *ws = device_scratch();
    if (!ws) return QSA_ERR_DEVICE;
    return qsa_forward(dims, q, k, v, routes, scale, out, out_fp32, lse, ws, kScratchBytes, stream);
}

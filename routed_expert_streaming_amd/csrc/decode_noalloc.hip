// moe_decode_forward_noalloc: the persistent decode driver with its
// workspace in a file-scope device array, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation).  Declaration and contract in include/moe.h.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_internal.h"

namespace moe {
int fail(int code, const char *fmt, ...);
int hip_fail(hipError_t e, const char *what);
}  // namespace moe

using namespace moe;

namespace {
// The decode workspace of every no-alloc call on a device: counters, the
// step-tagged exchange buffers, h and the layer table (no profiling stamps).
// Each device holds its own copy, from the library's load until the process
// ends.  In host code `scratch` names a host-side stand-in, not the device
// address: the address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the
// first call on each device, with that device current).
int scratch_for_current_device(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_E_INVAL, "device %d beyond the %d this library tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(MOE_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}
}  // namespace

namespace moe {
int decode_noalloc_scratch(void **out) { return scratch_for_current_device(out); }
}  // namespace moe

extern "C" int moe_decode_forward_noalloc(const moe_layer *layers, int32_t n_layers, const float *x, int32_t T,
                                          float *out, int32_t *idx_out, void *hip_stream) {
    int rc = decode_check_args(layers, n_layers, x, T, out);
    if (rc || T == 0) return rc;
    size_t need = 0;
    rc = decode_ws_bytes(layers, n_layers, /*stamps=*/false, &need);
    if (rc) return rc;
    if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
        return fail(MOE_E_SPACE,
                    "moe_decode_forward_noalloc: these layers need %zu bytes of decode workspace, above the %d bytes "
                    "of the library's scratch array (use moe_decode_forward with a caller workspace)",
                    need, MOE_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    rc = scratch_for_current_device(&ws);
    if (rc) return rc;
    return decode_forward_impl(layers, n_layers, x, T, out, idx_out, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES,
                               /*stamps=*/false, (hipStream_t)hip_stream);
}

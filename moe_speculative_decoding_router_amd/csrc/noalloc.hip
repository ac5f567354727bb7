// moe_verify_layer_noalloc: the verify call for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  The workspace of the call is a
// file-scope device array, one per GPU the library runs on, held until the
// process ends.  The kernels are those of moe_verify_layer; they take the
// array's device address as their workspace, exactly as they take a caller's
// buffer.
#include <hip/hip_runtime.h>

#include <atomic>

#include "internal.h"

namespace {

// The workspace of every no-allocation call on a device.  In host code the
// name `scratch` is only a host-side stand-in: the device address comes from
// hipGetSymbolAddress and is what every kernel argument and copy uses.
__device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// Device address of this device's array, looked up once per device (with
// that device current) and kept.
hipError_t scratch_ptr(void **out) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!p || (reinterpret_cast<uintptr_t>(p) & 255)) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev].store(p, std::memory_order_release);  // racing first calls store the same value
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

extern "C" int moe_verify_layer_noalloc(const moe_layer *layer, const float *x, int32_t T, const moe_bias *bias,
                                        float *y, moe_aux *aux, void *stream) {
    size_t need = 0;
    const int rc = moe::verify_needs(layer, T, bias, &need);
    if (rc != MOE_OK) return rc;
    if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) {
        char msg[160];
        snprintf(msg, sizeof(msg), "the call needs %zu bytes of workspace; the no-allocation array holds %zu",
                 need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
        return moe::set_error(MOE_EWORKSPACE, msg);
    }
    void *ws = nullptr;
    const hipError_t err = scratch_ptr(&ws);
    if (err != hipSuccess) {
        char msg[160];
        snprintf(msg, sizeof(msg), "device address of the workspace array: %s", hipGetErrorString(err));
        return moe::set_error(MOE_EHIP, msg);
    }
    return moe_verify_layer(layer, x, T, bias, y, aux, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}

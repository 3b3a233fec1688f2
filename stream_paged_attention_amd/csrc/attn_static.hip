// tf_attn_static: tf_attn_rows + tf_attn_merge with the split partials in a
// library-owned device array instead of a caller workspace, for callers that
// cannot allocate.  The kernels are the ones tf_attn_rows and tf_attn_merge
// launch; only where the partial records live differs.
#include <stdint.h>
#include <string.h>

#include <atomic>

#include <hip/hip_runtime.h>

#include "tf_attn.h"

// The partial records of every call on a device.  Each device that runs the
// library holds its own copy, for the life of the process.
static __device__ __align__(256) float scratch[TF_STATIC_PARTIALS_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;

// scratch's device address, per device (0 until that device's first call).
// The name `scratch` in host code is a host-side stand-in, not a device
// address: kernels get the address hipGetSymbolAddress returns.
std::atomic<uintptr_t> g_scratch[kMaxDevices];

// The scratch address on the current device, looked up once per device.
float *device_scratch()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    uintptr_t p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == 0) {
        void *addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr)
            return nullptr;
        p = reinterpret_cast<uintptr_t>(addr);
        // two threads may both look it up; they store the same address
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return reinterpret_cast<float *>(p);
}

}  // namespace

extern "C" int tf_attn_static(const tf_attn_args *a, hipStream_t stream)
{
    if (a == nullptr)
        return TF_E_INVALID;
    if (a->partials != nullptr)
        return TF_E_INVALID;   // the records go to the library's array
    if (a->partials_bytes > TF_STATIC_PARTIALS_BYTES)
        return TF_E_WORKSPACE;
    tf_attn_args b;
    memcpy(&b, a, sizeof b);
    if (a->split_keys > 0 && a->n_segments > 0) {
        float *p = device_scratch();
        if (p == nullptr)
            return TF_E_LAUNCH;
        b.partials = p;
    }
    int rc = tf_attn_rows(&b, stream);
    if (rc != TF_OK || a->split_keys == 0)
        return rc;
    return tf_attn_merge(&b, stream);
}

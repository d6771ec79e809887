// convrot_linear_noalloc: convrot_linear with the library's own device array
// as its workspace, for callers that cannot allocate (declared in
// include/convrot.h).
//
// The array is a file-scope device variable: every GPU the library runs on
// gets its own copy when the code object is loaded there, at its own address.
// In host code the variable's name is only a host-side stand-in, so its
// device address is looked up with hipGetSymbolAddress, once per device with
// that device current, and only that address is passed to the kernels.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "../../include/convrot.h"
#include "kernels.h"

namespace {

static __device__ __align__(256) uint8_t scratch[CONVROT_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices];   // device address of `scratch` per device (null until looked up)

// The current device's copy of `scratch`: CONVROT_OK and *out set, or
// CONVROT_ERR_LAUNCH if the device or the symbol cannot be resolved.
int device_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CONVROT_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CONVROT_ERR_LAUNCH;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return CONVROT_OK;
}

}  // namespace

extern "C" int convrot_linear_noalloc(const uint16_t* x, int64_t m, int64_t k, const int8_t* q_w,
                                      const float* s_w, int64_t n, uint16_t* y, void* stream) {
    // sizes and pointers first, as convrot_linear checks them (no HIP call)
    int st = convrot::linear_args(x, m, k, q_w, s_w, n, n, y);
    if (st != CONVROT_OK) return st;
    if (m == 0 || n == 0) return CONVROT_OK;
    const size_t need = convrot_workspace_bytes(m, k);
    if (need > CONVROT_NOALLOC_SCRATCH_BYTES) return CONVROT_ERR_SCRATCH;
    void* ws = nullptr;
    if ((st = device_scratch(&ws)) != CONVROT_OK) return st;
    return convrot::linear_common(x, m, k, q_w, s_w, n, n, y, ws, CONVROT_NOALLOC_SCRATCH_BYTES, false, stream);
}

// gdn_noalloc.hip -- gdn_layer_decode_noalloc: the layer decode step (gdn_layer_decode) with
// its intermediate tensors in a scratch array that the library holds in device memory, for
// callers that cannot allocate (code under HIP graph capture, serving loops that forbid
// allocation).  The caller passes inputs and outputs only.
//
// The scratch is a file-scope device array of kScratchBytes (64 MiB, held on each GPU the
// library is loaded on until the process ends).  Host code never uses the array's name as an
// address: on the first call on a device, with that device current, its device address is
// looked up with hipGetSymbolAddress and kept per device; kernels receive that address as
// their workspace.  Every call on a device shares the one array, so calls that overlap on one
// device (two streams, or two threads) race; calls ordered on one stream do not.  Nothing in
// the layer decode's workspace needs to start at zero: each call writes every intermediate
// before reading it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn.h"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;

__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up once per device).
hipError_t scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

int gdn_layer_decode_noalloc(const void *hidden, const void *w_in, const void *conv_w, const void *gamma,
                             const void *w_out, void *conv_state, float *state, void *out, float scale,
                             float l2_eps, float norm_eps, int B, int E, int Hk, int Hv, int dk, int dv, int order,
                             void *stream) {
    try {
        // sizes whose intermediates do not fit the scratch are refused before anything runs
        // (a shape the layer decode rejects reports 0 here and its own error below)
        if (gdn_layer_decode_workspace_size(B, E, Hk, Hv, dk, dv) > kScratchBytes) return GDN_ERR_WORKSPACE;
        void *ws = nullptr;
        if (scratch_address(&ws) != hipSuccess) return GDN_ERR_HIP;
        return gdn_layer_decode(hidden, w_in, conv_w, gamma, w_out, conv_state, state, out, scale, l2_eps, norm_eps,
                                B, E, Hk, Hv, dk, dv, order, ws, kScratchBytes, stream);
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

}  // extern "C"

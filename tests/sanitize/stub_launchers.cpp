// stub_launchers.cpp -- host stand-ins for the kernel launchers declared in gdn_launch.hpp,
// so the C-ABI layer (gdn_api.cpp) can be built and run on a CPU under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Test infrastructure: nothing here is part of the library.
// Every launcher records that it was reached and returns success; the shape predicates
// restate the library's documented rules (chunked MFMA path: dk = dv in {64, 128}; chunked
// fp32 path: dk, dv in {16, 32, 64}; gate columns 2 Hv <= 64).
#include <cstring>

#include "gdn_launch.hpp"

int g_launches = 0;   // read by the driver

namespace gdn {
hipError_t launch_prep(const PrepArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_conv_state_out(const PrepArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode(const DecodeArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_gated_rmsnorm(const NormArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_proj(const ProjArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
bool proj_gates_supported(int heads) { return 2 * heads <= 64; }
int device_cus() { return 256; }
hipError_t launch_prefill_recurrent(const PrefillArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
bool chunked_f32_supported(int dk, int dv) {
    return (dk == 16 || dk == 32 || dk == 64) && (dv == 16 || dv == 32 || dv == 64);
}
hipError_t launch_prefill_chunked_f32(const PrefillArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
bool chunked_supported(int dk, int dv) { return dk == dv && (dk == 64 || dk == 128); }
size_t chunked_workspace_bytes(int T, int N, int Hv, int dk, int dv) {
    (void)dv;
    return kWsHeader + ((size_t)T / 64 + (size_t)N) * (size_t)Hv * ((size_t)dk * 1024 + 256) +
           (size_t)N * Hv * dk * dk * 4;
}
size_t norm_epi_words(int T, int N, int Hv, int dv) { return ((size_t)T / 64 + (size_t)N) * (size_t)Hv * (dv / 32) * 64; }
hipError_t launch_prefill_chunked(const PrefillArgs &, hipStream_t, int) { ++g_launches; return hipSuccess; }
hipError_t workspace_status(void *ws, hipStream_t, unsigned long long *word, bool clear) {
    std::memcpy(word, ws, sizeof(*word));   // host memory stands in for the workspace
    if (clear) std::memset(ws, 0, sizeof(*word));
    return hipSuccess;
}
hipError_t copy_seqlens(const int32_t *cu, int n, hipStream_t, int32_t *host) {
    std::memcpy(host, cu, sizeof(int32_t) * (size_t)n);
    return hipSuccess;
}
}  // namespace gdn

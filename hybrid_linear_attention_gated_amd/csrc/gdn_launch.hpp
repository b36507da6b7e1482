// gdn_launch.hpp -- host-side launch entry points of the kernels (one per
// translation unit).  Arguments are validated by gdn_api.cpp before any of
// these is called; each returns the first HIP error it meets.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Workspace status word of the chunked prefill (see gdn_prefill_workspace_status in gdn.h):
// (kStatusTag << 32) | status code, stored by a kernel that meets a failure.
constexpr unsigned kStatusTag = 0x67646e73u;
constexpr unsigned kStatusTimeout = 8;     // GDN_ERR_TIMEOUT
constexpr unsigned kStatusNonFinite = 9;   // GDN_ERR_NONFINITE
// Header at the start of the chunked prefill's workspace: the status word (8 bytes), then
// an optional bound on the state pass's record waits ((kSpinTag << 32) | iterations; any
// other value means the default, about a second).
constexpr size_t kWsHeader = 256;
constexpr unsigned kSpinTag = 0x7370696eu;

struct PrepArgs {
    const void *x, *w;
    const int32_t *cu;
    int N;
    const void *cs_in;
    void *cs_out;
    float *q, *k, *v;
    int T, Hk, Hv, dk, dv;
    bool bf16;   // element type of x / conv_w / conv states
    float eps;
};

// Pre-conv inputs of the fused prefill (gdn_prefill): the chunk-local kernel runs the conv
// prep itself, and q, k, v of PrefillArgs are unused.
struct FusedPrep {
    const void *x, *w;
    const void *cs_in;
    void *cs_out;
    bool bf16;   // element type of x / conv_w / conv states
    float eps;
    bool w_bf16 = false;   // with bf16 false: conv_w is bf16 while x and the conv states are fp32
};

// Gated RMSNorm epilogue formed inside the prefill (the layer's prefill): out = o *
// rsqrt(mean o^2 + eps) * gamma * SiLU(z) per (token, value head) row of dv channels ([T][Hv dv]
// rows; z fp16, gamma and out bf16).  `sums` holds the row-sum words the
// workgroups of a head exchange (norm_epi_words of them).  The launcher applies it where
// its schedule can (and then sets `fused`); otherwise the caller runs the separate
// epilogue over o.
struct NormEpi {
    const void *z, *gamma;
    void *out;
    float eps;
    unsigned long long *sums;
    bool fused = false;
};
// 64-bit words NormEpi::sums needs for T tokens in N sequences and Hv value heads of dv channels
size_t norm_epi_words(int T, int N, int Hv, int dv);

struct PrefillArgs {
    const float *q, *k, *v;
    const float *g, *beta;
    const int32_t *cu;
    int N;
    const float *s0;
    float *sf;
    float *o;
    float scale;
    int T, Hk, Hv, dk, dv;
    void *ws;
    size_t ws_bytes;
    const FusedPrep *fp = nullptr;   // set: fused prep (chunked path only)
    int order = 0;                   // 0: decay before the retrieval, 1: retrieval from the undecayed state
    NormEpi *norm = nullptr;         // set: the gated RMSNorm epilogue where the schedule allows it
};

struct DecodeArgs {
    const void *x, *w;
    void *cs;
    const float *g, *beta;
    float *state;
    float *o;
    float scale, eps;
    int B, Hk, Hv, dk, dv;
    bool bf16;
    int order = 0;   // as in PrefillArgs
    // gated output (gdn_decode_step_gated): when `out` is set, out = RMSNorm(o) * gamma *
    // SiLU(z) in the element type is written instead of o
    const void *z = nullptr, *gamma = nullptr;
    void *out = nullptr;
    float norm_eps = 0.f;
    // the layer's decode: x and the conv cache fp32, conv weights, z and out bf16 (gated only)
    bool layer_types = false;
};

struct NormArgs {
    const float *y;
    const void *z, *gamma;
    void *out;
    long rows;
    int dv;
    float eps;
    bool bf16;   // element type of z / gamma / out
    bool z_f16 = false;   // with bf16: z is fp16 (the layer prefill's gate), gamma and out bf16
};

// y = a w^T on bf16 MFMA (a [M][K], w [N + 2 heads][K], bf16): columns n < n_split go to
// y0[m][n] (row length ld0), the others to y1[m][n - n_split] (row length ld1); with
// heads > 0 the 2 heads rows of w after row N give g[m][h] = -softplus and
// beta[m][h] = sigmoid of their products.  K % 64 == 0, N % 4 == 0, 2 heads <= 64.
struct ProjArgs {
    const void *a, *w;
    int M, N, K;
    void *y0;
    int ld0, n_split;
    void *y1;
    int ld1;
    float *g = nullptr, *beta = nullptr;
    int heads = 0;
    // optional fp32 buffer of partial_cap floats: with few tiles (and no gate columns) the
    // launcher splits k and sums the slices' planes in a second pass
    float *partial = nullptr;
    size_t partial_cap = 0;
    // the layer's input projection: columns n < n_split go to y0 as fp32 (and with y1_f16, the
    // others to y1 as fp16, clamped to its range: the layer prefill's gate z)
    bool y0_f32 = false;
    bool y1_f16 = false;
    int tiles_m = 0, tiles_n = 0, ntiles = 0, ksplit = 1;   // set by the launcher
};

hipError_t launch_prep(const PrepArgs &a, hipStream_t st);
// conv_state_out[s] = last three inputs of sequence s (a launch of its own)
hipError_t launch_conv_state_out(const PrepArgs &a, hipStream_t st);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t st);
// gated RMSNorm epilogue over rows of dv channels (dv in {16, 32, 64, 128, 256})
hipError_t launch_gated_rmsnorm(const NormArgs &a, hipStream_t st);

hipError_t launch_proj(const ProjArgs &a, hipStream_t st);
bool proj_gates_supported(int heads);
// compute units of the current device (cached per device; 0 if unknown)
int device_cus();

// token-recurrent fp32 path (GDN_F32 and the small head dims)
hipError_t launch_prefill_recurrent(const PrefillArgs &a, hipStream_t st);

// chunked (WY / UT) form in fp32 for dk, dv in {16, 32, 64} (GDN_MATH_F32_CHUNKED)
bool chunked_f32_supported(int dk, int dv);
hipError_t launch_prefill_chunked_f32(const PrefillArgs &a, hipStream_t st);

// chunked MFMA path (dk = dv in {64, 128})
bool chunked_supported(int dk, int dv);
size_t chunked_workspace_bytes(int T, int N, int Hv, int dk, int dv);
// phases: bit 0 = chunk-local kernel, bit 1 = state-pass kernel
hipError_t launch_prefill_chunked(const PrefillArgs &a, hipStream_t st, int phases);
// the chunked prefill workspace's status word, read after `st` and the library's second
// stream have drained (reset to 0 with `clear`)
hipError_t workspace_status(void *ws, hipStream_t st, unsigned long long *word, bool clear);
// n int32 of device memory to the host, synchronously on `st`
hipError_t copy_seqlens(const int32_t *cu, int n, hipStream_t st, int32_t *host);

}  // namespace gdn

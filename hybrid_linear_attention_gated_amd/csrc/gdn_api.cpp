// gdn_api.cpp -- the extern "C" entry points declared in include/gdn.h:
// argument validation on the host (nothing is enqueued when it fails), pointer
// overlap checks, and dispatch to the kernels' launchers.
#include "gdn.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <vector>

#include "gdn_launch.hpp"

namespace {

bool valid_dtype(int dt) { return dt == GDN_F32 || dt == GDN_BF16; }
size_t elem_bytes(int dt) { return dt == GDN_BF16 ? 2 : 4; }
bool pow2_in(int d, int lo, int hi) { return d >= lo && d <= hi && (d & (d - 1)) == 0; }

struct Range {
    const void *p;
    size_t bytes;
};

bool overlap(Range a, Range b) {
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + a.bytes;
    const uintptr_t b0 = (uintptr_t)b.p, b1 = b0 + b.bytes;
    return a0 < b1 && b0 < a1;
}

// Exact aliasing is allowed where documented; partial overlap never is.
bool bad_partial_alias(Range a, Range b) { return overlap(a, b) && !(a.p == b.p && a.bytes == b.bytes); }

// Size limits that keep every byte count the checks below form within 64 bits (tensor
// sizes are products of up to five of these with int token counts): heads, sequences or
// decode rows, and rows of the standalone norm.
constexpr int kMaxHeads = 4096;
constexpr int kMaxSeqs = 1 << 24;
constexpr long kMaxNormRows = 1L << 40;

int check_heads(int Hk, int Hv) {
    if (Hk <= 0 || Hv <= 0 || Hv % Hk != 0 || Hk > kMaxHeads || Hv > kMaxHeads) return GDN_ERR_BAD_SHAPE;
    return GDN_OK;
}

int check_seqs(const int32_t *cu, int N, int T) {
    if (T < 0 || N < 1 || N > kMaxSeqs) return GDN_ERR_BAD_SHAPE;
    if (!cu && N != 1) return GDN_ERR_BAD_SHAPE;
    return GDN_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

bool valid_order(int order) { return order == GDN_ORDER_DECAY_FIRST || order == GDN_ORDER_RETRIEVE_FIRST; }

static_assert(gdn::kStatusTimeout == GDN_ERR_TIMEOUT && gdn::kStatusNonFinite == GDN_ERR_NONFINITE,
              "device status codes are the ABI's");

// GDN_DEBUG_CHECK set (and not "0") in the environment when the library first looks:
// prefill calls then check cu_seqlens on the host before launching and wait for their own
// completion to return the workspace status (timeout, non-finite output).
bool debug_check() {
    static const bool on = [] {
        const char *v = std::getenv("GDN_DEBUG_CHECK");
        return v && *v && std::strcmp(v, "0") != 0;
    }();
    return on;
}

// The debug check of cu_seqlens: cu[0] = 0, non-decreasing, cu[N] = T.
int check_seqlens_on_host(const int32_t *cu, int N, int T, hipStream_t st) {
    if (!cu) return GDN_OK;
    std::vector<int32_t> h((size_t)N + 1);
    if (gdn::copy_seqlens(cu, N + 1, st, h.data()) != hipSuccess) return GDN_ERR_HIP;
    if (h[0] != 0 || h[(size_t)N] != T) return GDN_ERR_BAD_SHAPE;
    for (int i = 0; i < N; ++i)
        if (h[(size_t)i + 1] < h[(size_t)i]) return GDN_ERR_BAD_SHAPE;
    return GDN_OK;
}

// The status of a chunked prefill's workspace (its header word), cleared as it is read.
int take_status(void *ws, hipStream_t st) {
    unsigned long long w = 0;
    if (gdn::workspace_status(ws, st, &w, true) != hipSuccess) return GDN_ERR_HIP;
    return (unsigned)(w >> 32) == gdn::kStatusTag ? (int)(w & 0xffffffffu) : GDN_OK;
}

// Every non-NULL device pointer is 16-byte aligned (the kernels move 16-byte vectors).
bool aligned16(std::initializer_list<const void *> ptrs) {
    for (const void *p : ptrs)
        if (reinterpret_cast<uintptr_t>(p) & 15) return false;
    return true;
}

}  // namespace

extern "C" {

const char *gdn_status_string(int status) {
    switch (status) {
        case GDN_OK: return "GDN_OK";
        case GDN_ERR_NULL_POINTER: return "GDN_ERR_NULL_POINTER: a required pointer is NULL";
        case GDN_ERR_BAD_SHAPE: return "GDN_ERR_BAD_SHAPE: inconsistent or negative sizes";
        case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: head dim / dtype combination not implemented";
        case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
        case GDN_ERR_HIP: return "GDN_ERR_HIP: a HIP launch or runtime call failed";
        case GDN_ERR_ALIAS: return "GDN_ERR_ALIAS: an output overlaps an input it must not overlap";
        case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN: a device pointer is not 16-byte aligned";
        case GDN_ERR_TIMEOUT:
            return "GDN_ERR_TIMEOUT: the state pass stopped waiting for a chunk's record; outputs are NaN";
        case GDN_ERR_NONFINITE: return "GDN_ERR_NONFINITE: an output or final state is inf or NaN";
        default: return "unknown gdn status";
    }
}

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

int gdn_conv_qk_prep(const void *x, const void *conv_w, const int32_t *cu_seqlens, int N,
                     const void *conv_state_in, void *conv_state_out, float *q, float *k, float *v, int T, int Hk,
                     int Hv, int dk, int dv, int dtype, float l2_eps, void *stream) {
    try {
        if (int e = check_seqs(cu_seqlens, N, T)) return e;
        if (!conv_w || (T > 0 && (!x || !q || !k || !v))) return GDN_ERR_NULL_POINTER;
        if (!aligned16({x, conv_w, cu_seqlens, conv_state_in, conv_state_out, q, k, v})) return GDN_ERR_ALIGN;
        if (int e = check_heads(Hk, Hv)) return e;
        if (!valid_dtype(dtype)) return GDN_ERR_UNSUPPORTED;
        if (!pow2_in(dk, 16, 256) || dv < 8 || dv > 256 || dv % 8 != 0) return GDN_ERR_UNSUPPORTED;
        if (!(l2_eps >= 0.f) || !std::isfinite(l2_eps)) return GDN_ERR_BAD_SHAPE;
        const size_t eb = elem_bytes(dtype);
        const size_t conv_dim = 2 * (size_t)Hk * dk + (size_t)Hv * dv;
        const Range rx{x, (size_t)T * conv_dim * eb}, rw{conv_w, conv_dim * 4 * eb};
        const Range rci{conv_state_in, (size_t)N * 3 * conv_dim * eb}, rco{conv_state_out, rci.bytes};
        const Range rq{q, (size_t)T * Hk * dk * 4}, rk{k, rq.bytes}, rv{v, (size_t)T * Hv * dv * 4};
        for (Range out : {rq, rk, rv})
            for (Range in : {rx, rw, rci})
                if (overlap(out, in)) return GDN_ERR_ALIAS;
        if (overlap(rco, rx) || overlap(rco, rw) || bad_partial_alias(rco, rci)) return GDN_ERR_ALIAS;
        if (overlap(rq, rk) || overlap(rq, rv) || overlap(rk, rv) || overlap(rco, rq) || overlap(rco, rk) ||
            overlap(rco, rv))
            return GDN_ERR_ALIAS;
        gdn::PrepArgs a{x, conv_w, cu_seqlens, N, conv_state_in, conv_state_out, q, k, v,
                        T, Hk, Hv, dk, dv, dtype == GDN_BF16, l2_eps};
        return hip_status(gdn::launch_prep(a, (hipStream_t)stream));
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

size_t gdn_chunk_prefill_workspace_size(int T, int N, int Hk, int Hv, int dk, int dv, int math) {
    if (T < 0 || N < 1 || N > kMaxSeqs || check_heads(Hk, Hv) != GDN_OK) return 0;
    if (math != GDN_MATH_MFMA || !gdn::chunked_supported(dk, dv)) return 0;
    return gdn::chunked_workspace_bytes(T, N, Hv, dk, dv);
}

namespace {

// Shared validation + dispatch of gdn_chunk_prefill and its two phases.
int chunk_prefill_impl(const float *q, const float *k, const float *v, const float *g, const float *beta,
                       const int32_t *cu_seqlens, int N, const float *initial_state, float *final_state, float *o,
                       float scale, int T, int Hk, int Hv, int dk, int dv, int math, int order, void *workspace,
                       size_t workspace_bytes, void *stream, int phases) {
    try {
        if (int e = check_seqs(cu_seqlens, N, T)) return e;
        const bool need_inputs = phases & 1, need_outputs = phases & 2;
        if (T > 0 && need_inputs && (!q || !k || !v || !g || !beta)) return GDN_ERR_NULL_POINTER;
        if (T > 0 && need_outputs && !o) return GDN_ERR_NULL_POINTER;
        if (!aligned16({q, k, v, g, beta, cu_seqlens, initial_state, final_state, o, workspace})) return GDN_ERR_ALIGN;
        if (int e = check_heads(Hk, Hv)) return e;
        if (math != GDN_MATH_F32 && math != GDN_MATH_MFMA && math != GDN_MATH_F32_CHUNKED) return GDN_ERR_UNSUPPORTED;
        if (!valid_order(order)) return GDN_ERR_UNSUPPORTED;
        if (phases != 3 && math != GDN_MATH_MFMA) return GDN_ERR_UNSUPPORTED;
        if (!pow2_in(dk, 16, 128) || !pow2_in(dv, 16, 128)) return GDN_ERR_UNSUPPORTED;
        if (math == GDN_MATH_MFMA && !gdn::chunked_supported(dk, dv)) return GDN_ERR_UNSUPPORTED;
        if (math == GDN_MATH_F32_CHUNKED && !gdn::chunked_f32_supported(dk, dv)) return GDN_ERR_UNSUPPORTED;
        if (!std::isfinite(scale)) return GDN_ERR_BAD_SHAPE;
        const bool chunked = math == GDN_MATH_MFMA;
        const size_t need = chunked ? gdn::chunked_workspace_bytes(T, N, Hv, dk, dv) : 0;
        if (need > 0 && (!workspace || workspace_bytes < need)) return GDN_ERR_WORKSPACE;
        const size_t st_bytes = (size_t)N * Hv * dk * dv * 4;
        const Range rq{q, (size_t)T * Hk * dk * 4}, rk{k, rq.bytes}, rv{v, (size_t)T * Hv * dv * 4};
        const Range rg{g, (size_t)T * Hv * 4}, rb{beta, rg.bytes}, rs0{initial_state, st_bytes},
            rsf{final_state, st_bytes}, ro{o, (size_t)T * Hv * dv * 4}, rws{workspace, need};
        for (Range in : {rq, rk, rv, rg, rb, rs0, rsf, rws})
            if (overlap(ro, in)) return GDN_ERR_ALIAS;
        for (Range in : {rq, rk, rv, rg, rb, rws})
            if (overlap(rsf, in)) return GDN_ERR_ALIAS;
        if (bad_partial_alias(rsf, rs0)) return GDN_ERR_ALIAS;
        for (Range in : {rq, rk, rv, rg, rb, rs0})
            if (overlap(rws, in)) return GDN_ERR_ALIAS;
        gdn::PrefillArgs a{q, k, v, g, beta, cu_seqlens, N, initial_state, final_state, o, scale,
                           T, Hk, Hv, dk, dv, workspace, workspace_bytes};
        a.order = order;
        hipStream_t st = (hipStream_t)stream;
        const bool dbg = debug_check();
        if (dbg) {
            if (int e = check_seqlens_on_host(cu_seqlens, N, T, st)) return e;
            if (chunked && (phases & 1)) (void)take_status(workspace, st);   // start from a clear status word
        }
        if (int e = hip_status(chunked                          ? gdn::launch_prefill_chunked(a, st, phases)
                               : math == GDN_MATH_F32_CHUNKED ? gdn::launch_prefill_chunked_f32(a, st)
                                                              : gdn::launch_prefill_recurrent(a, st)))
            return e;
        return dbg && chunked && (phases & 2) ? take_status(workspace, st) : GDN_OK;
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

}  // namespace

int gdn_chunk_prefill(const float *q, const float *k, const float *v, const float *g, const float *beta,
                      const int32_t *cu_seqlens, int N, const float *initial_state, float *final_state, float *o,
                      float scale, int T, int Hk, int Hv, int dk, int dv, int math, int order, void *workspace,
                      size_t workspace_bytes, void *stream) {
    return chunk_prefill_impl(q, k, v, g, beta, cu_seqlens, N, initial_state, final_state, o, scale, T, Hk, Hv, dk,
                              dv, math, order, workspace, workspace_bytes, stream, 3);
}

int gdn_chunk_prefill_local(const float *q, const float *k, const float *v, const float *g, const float *beta,
                            const int32_t *cu_seqlens, int N, float scale, int T, int Hk, int Hv, int dk, int dv,
                            int order, void *workspace, size_t workspace_bytes, void *stream) {
    return chunk_prefill_impl(q, k, v, g, beta, cu_seqlens, N, nullptr, nullptr, nullptr, scale, T, Hk, Hv, dk, dv,
                              GDN_MATH_MFMA, order, workspace, workspace_bytes, stream, 1);
}

int gdn_chunk_prefill_state(const int32_t *cu_seqlens, int N, const float *initial_state, float *final_state,
                            float *o, int T, int Hk, int Hv, int dk, int dv, const void *workspace,
                            size_t workspace_bytes, void *stream) {
    return chunk_prefill_impl(nullptr, nullptr, nullptr, nullptr, nullptr, cu_seqlens, N, initial_state, final_state,
                              o, 1.0f, T, Hk, Hv, dk, dv, GDN_MATH_MFMA, GDN_ORDER_DECAY_FIRST,
                              const_cast<void *>(workspace), workspace_bytes, stream, 2);
}

namespace {

// Shared validation + dispatch of gdn_prefill (phases 3) and gdn_prefill_local (phase 1).
// layer_types: the layer's prefill (x and the conv caches fp32, conv weights bf16; dtype
// is then ignored).
int prefill_impl(const void *x, const void *conv_w, const int32_t *cu_seqlens, int N, const void *conv_state_in,
                 void *conv_state_out, const float *g, const float *beta, const float *initial_state,
                 float *final_state, float *o, float scale, float l2_eps, int T, int Hk, int Hv, int dk, int dv,
                 int dtype, int order, void *workspace, size_t workspace_bytes, void *stream, int phases,
                 bool layer_types = false, gdn::NormEpi *norm = nullptr) {
    try {
        if (int e = check_seqs(cu_seqlens, N, T)) return e;
        if (!conv_w || (T > 0 && (!x || !g || !beta || ((phases & 2) && !o)))) return GDN_ERR_NULL_POINTER;
        if (!aligned16({x, conv_w, cu_seqlens, conv_state_in, conv_state_out, g, beta, initial_state, final_state, o,
                        workspace}))
            return GDN_ERR_ALIGN;
        if (int e = check_heads(Hk, Hv)) return e;
        if (!valid_dtype(dtype) || !valid_order(order)) return GDN_ERR_UNSUPPORTED;
        if (!gdn::chunked_supported(dk, dv)) return GDN_ERR_UNSUPPORTED;
        if (!(l2_eps >= 0.f) || !std::isfinite(l2_eps) || !std::isfinite(scale)) return GDN_ERR_BAD_SHAPE;
        const size_t need = gdn::chunked_workspace_bytes(T, N, Hv, dk, dv);
        if (!workspace || workspace_bytes < need) return GDN_ERR_WORKSPACE;
        const size_t eb = layer_types ? 4 : elem_bytes(dtype), wb = layer_types ? 2 : eb;
        const size_t conv_dim = 2 * (size_t)Hk * dk + (size_t)Hv * dv;
        const size_t st_bytes = (size_t)N * Hv * dk * dv * 4;
        const Range rx{x, (size_t)T * conv_dim * eb}, rw{conv_w, conv_dim * 4 * wb};
        const Range rci{conv_state_in, (size_t)N * 3 * conv_dim * eb}, rco{conv_state_out, rci.bytes};
        const Range rg{g, (size_t)T * Hv * 4}, rb{beta, rg.bytes}, rs0{initial_state, st_bytes},
            rsf{final_state, st_bytes}, ro{o, (size_t)T * Hv * dv * 4}, rws{workspace, need};
        for (Range in : {rx, rw, rci, rco, rg, rb, rs0, rsf, rws})
            if (overlap(ro, in)) return GDN_ERR_ALIAS;
        for (Range in : {rx, rw, rci, rco, rg, rb, rws})
            if (overlap(rsf, in)) return GDN_ERR_ALIAS;
        for (Range in : {rx, rw, rg, rb, rs0, rws})
            if (overlap(rco, in)) return GDN_ERR_ALIAS;
        for (Range in : {rx, rw, rci, rg, rb, rs0})
            if (overlap(rws, in)) return GDN_ERR_ALIAS;
        if (bad_partial_alias(rsf, rs0) || bad_partial_alias(rco, rci)) return GDN_ERR_ALIAS;
        const gdn::FusedPrep fp{x, conv_w, conv_state_in, conv_state_out, !layer_types && dtype == GDN_BF16, l2_eps,
                                layer_types};
        gdn::PrefillArgs a{nullptr, nullptr, nullptr, g, beta, cu_seqlens, N, initial_state, final_state, o, scale,
                           T, Hk, Hv, dk, dv, workspace, workspace_bytes, &fp};
        a.order = order;
        a.norm = norm;
        hipStream_t st = (hipStream_t)stream;
        const bool dbg = debug_check();
        if (dbg) {
            if (int e = check_seqlens_on_host(cu_seqlens, N, T, st)) return e;
            (void)take_status(workspace, st);   // start from a clear status word
        }
        if (int e = hip_status(gdn::launch_prefill_chunked(a, st, phases))) return e;
        return dbg && (phases & 2) ? take_status(workspace, st) : GDN_OK;
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

}  // namespace

int gdn_prefill(const void *x, const void *conv_w, const int32_t *cu_seqlens, int N, const void *conv_state_in,
                void *conv_state_out, const float *g, const float *beta, const float *initial_state,
                float *final_state, float *o, float scale, float l2_eps, int T, int Hk, int Hv, int dk, int dv,
                int dtype, int order, void *workspace, size_t workspace_bytes, void *stream) {
    return prefill_impl(x, conv_w, cu_seqlens, N, conv_state_in, conv_state_out, g, beta, initial_state,
                        final_state, o, scale, l2_eps, T, Hk, Hv, dk, dv, dtype, order, workspace, workspace_bytes,
                        stream, 3);
}

int gdn_prefill_workspace_status(void *workspace, size_t workspace_bytes, void *stream) {
    try {
        if (!workspace) return GDN_ERR_NULL_POINTER;
        if (!aligned16({workspace})) return GDN_ERR_ALIGN;
        if (workspace_bytes < gdn::kWsHeader) return GDN_ERR_WORKSPACE;
        return take_status(workspace, (hipStream_t)stream);
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

int gdn_prefill_local(const void *x, const void *conv_w, const int32_t *cu_seqlens, int N,
                      const void *conv_state_in, void *conv_state_out, const float *g, const float *beta,
                      float scale, float l2_eps, int T, int Hk, int Hv, int dk, int dv, int dtype, int order,
                      void *workspace, size_t workspace_bytes, void *stream) {
    return prefill_impl(x, conv_w, cu_seqlens, N, conv_state_in, conv_state_out, g, beta, nullptr, nullptr, nullptr,
                        scale, l2_eps, T, Hk, Hv, dk, dv, dtype, order, workspace, workspace_bytes, stream, 1);
}

namespace {

// Shared validation + dispatch of gdn_decode_step and gdn_decode_step_gated (z, gamma, out set).
int decode_impl(const void *x, const void *conv_w, void *conv_state, const float *g, const float *beta,
                float *state, float *o, const void *z, const void *gamma, void *out, float scale, float l2_eps,
                float norm_eps, int B, int Hk, int Hv, int dk, int dv, int dtype, int order, void *stream) {
    try {
        const bool gated = out != nullptr || z != nullptr || gamma != nullptr;
        if (B < 0 || B > kMaxSeqs) return GDN_ERR_BAD_SHAPE;
        if (!conv_w || (B > 0 && (!x || !conv_state || !g || !beta || !state))) return GDN_ERR_NULL_POINTER;
        if (gated ? (!gamma || (B > 0 && (!z || !out))) : (B > 0 && !o)) return GDN_ERR_NULL_POINTER;
        if (!aligned16({x, conv_w, conv_state, g, beta, state, o, z, gamma, out})) return GDN_ERR_ALIGN;
        if (int e = check_heads(Hk, Hv)) return e;
        if (!valid_dtype(dtype) || !valid_order(order)) return GDN_ERR_UNSUPPORTED;
        if (!pow2_in(dk, 16, 128) || !pow2_in(dv, 16, 128)) return GDN_ERR_UNSUPPORTED;
        if (!std::isfinite(scale) || !(l2_eps >= 0.f) || !std::isfinite(l2_eps)) return GDN_ERR_BAD_SHAPE;
        if (gated && (!(norm_eps >= 0.f) || !std::isfinite(norm_eps))) return GDN_ERR_BAD_SHAPE;
        const size_t eb = elem_bytes(dtype);
        const size_t conv_dim = 2 * (size_t)Hk * dk + (size_t)Hv * dv;
        const Range rx{x, (size_t)B * conv_dim * eb}, rw{conv_w, conv_dim * 4 * eb},
            rcs{conv_state, (size_t)B * 3 * conv_dim * eb}, rg{g, (size_t)B * Hv * 4}, rb{beta, rg.bytes},
            rst{state, (size_t)B * Hv * dk * dv * 4}, ro{gated ? nullptr : o, (size_t)B * Hv * dv * 4},
            rz{z, (size_t)B * Hv * dv * eb}, rgm{gamma, (size_t)dv * eb}, rout{out, rz.bytes};
        for (Range res : {ro, rout})
            for (Range in : {rx, rw, rcs, rg, rb, rst, rz, rgm})
                if (overlap(res, in)) return GDN_ERR_ALIAS;
        for (Range in : {rx, rw, rg, rb, rz, rgm})
            if (overlap(rcs, in) || overlap(rst, in)) return GDN_ERR_ALIAS;
        if (overlap(rcs, rst)) return GDN_ERR_ALIAS;
        gdn::DecodeArgs a{x, conv_w, conv_state, g, beta, state, o, scale, l2_eps, B, Hk, Hv, dk, dv,
                          dtype == GDN_BF16};
        a.order = order;
        if (gated) {
            a.z = z;
            a.gamma = gamma;
            a.out = out;
            a.norm_eps = norm_eps;
        }
        return hip_status(gdn::launch_decode(a, (hipStream_t)stream));
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

}  // namespace

int gdn_decode_step(const void *x, const void *conv_w, void *conv_state, const float *g, const float *beta,
                    float *state, float *o, float scale, float l2_eps, int B, int Hk, int Hv, int dk, int dv,
                    int dtype, int order, void *stream) {
    if (!o && B > 0) return GDN_ERR_NULL_POINTER;
    return decode_impl(x, conv_w, conv_state, g, beta, state, o, nullptr, nullptr, nullptr, scale, l2_eps, 0.f, B,
                       Hk, Hv, dk, dv, dtype, order, stream);
}

int gdn_decode_step_gated(const void *x, const void *conv_w, void *conv_state, const float *g,
                          const float *beta, float *state, const void *z, const void *gamma, void *out,
                          float scale, float l2_eps, float norm_eps, int B, int Hk, int Hv, int dk, int dv,
                          int dtype, int order, void *stream) {
    if (!gamma || (B > 0 && (!z || !out))) return GDN_ERR_NULL_POINTER;
    return decode_impl(x, conv_w, conv_state, g, beta, state, nullptr, z, gamma, out, scale, l2_eps, norm_eps, B,
                       Hk, Hv, dk, dv, dtype, order, stream);
}

int gdn_gated_rmsnorm(const float *y, const void *z, const void *gamma, void *out, long rows, int dv,
                      float eps, int dtype, void *stream) {
    try {
        if (rows < 0 || rows > kMaxNormRows) return GDN_ERR_BAD_SHAPE;
        if (!gamma || (rows > 0 && (!y || !z || !out))) return GDN_ERR_NULL_POINTER;
        if (!aligned16({y, z, gamma, out})) return GDN_ERR_ALIGN;
        if (!valid_dtype(dtype)) return GDN_ERR_UNSUPPORTED;
        if (!pow2_in(dv, 16, 256)) return GDN_ERR_UNSUPPORTED;
        if (!(eps >= 0.f) || !std::isfinite(eps)) return GDN_ERR_BAD_SHAPE;
        const size_t eb = elem_bytes(dtype);
        const size_t n = (size_t)rows * dv;
        const Range ry{y, n * 4}, rz{z, n * eb}, rgm{gamma, (size_t)dv * eb}, rout{out, n * eb};
        // out may replace y (fp32) or z exactly: each element is read before it is written,
        // by the same thread
        if (overlap(rout, rgm)) return GDN_ERR_ALIAS;
        if (bad_partial_alias(rout, ry) || bad_partial_alias(rout, rz)) return GDN_ERR_ALIAS;
        gdn::NormArgs a{y, z, gamma, out, rows, dv, eps, dtype == GDN_BF16};
        return hip_status(gdn::launch_gated_rmsnorm(a, (hipStream_t)stream));
    } catch (...) {
        return GDN_ERR_HIP;
    }
}


namespace {

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Host checks shared by the projections: K a positive multiple of 64 (the k-stage depth)
// and at most 2^20 (a tile's 256 rows then span < 2^31 bytes, the reach of the kernel's
// 32-bit buffer offsets), output row lengths multiples of 4 (8-byte stores of 4 bf16).
constexpr int kProjMaxK = 1 << 20;
bool proj_shape_ok(int M, int N, int K) {
    return M >= 0 && N > 0 && N % 4 == 0 && K > 0 && K % 64 == 0 && K <= kProjMaxK;
}

// x_f32: the layer's input projection (x fp32); otherwise the public one (x bf16).
// x_f32: x leaves in fp32 (the layer calls); z_f16: z in fp16 (the layer prefill)
int in_proj_impl(const void *hidden, const void *w_in, void *x, void *z, float *g, float *beta, int T, int E,
                 int Hk, int Hv, int dk, int dv, hipStream_t st, bool x_f32 = false, bool z_f16 = false) {
    const size_t C = 2 * (size_t)Hk * dk + (size_t)Hv * dv, Z = (size_t)Hv * dv;
    gdn::ProjArgs a{hidden, w_in, T, (int)(C + Z), E, x, (int)C, (int)C, z, (int)Z};
    a.g = g;
    a.beta = beta;
    a.heads = Hv;
    a.y0_f32 = x_f32;
    a.y1_f16 = x_f32 && z_f16;
    return hip_status(gdn::launch_proj(a, st));
}

// partial (optional, partial_cap floats): lets the launcher split k when the output has
// few tiles (the layer decode's output projection)
int linear_impl(const void *a, const void *w, void *y, int M, int N, int K, hipStream_t st,
                float *partial = nullptr, size_t partial_cap = 0) {
    gdn::ProjArgs p{a, w, M, N, K, y, N, N, nullptr, 0};
    p.partial = partial;
    p.partial_cap = partial_cap;
    return hip_status(gdn::launch_proj(p, st));
}

// k slices the layer decode's output projection may be split into (partial-sum planes)
constexpr int kDecodeProjSplits = 16;

// Shapes the layer entry points accept: the projections' k extents (E and Hv dv) are
// multiples of 64, the gate columns fit the gate workgroups, and dk, dv are 16-multiples.
int check_layer_shape(int E, int Hk, int Hv, int dk, int dv) {
    if (int e = check_heads(Hk, Hv)) return e;
    if (E <= 0) return GDN_ERR_BAD_SHAPE;
    if (E % 64 != 0 || ((size_t)Hv * dv) % 64 != 0 || !gdn::proj_gates_supported(Hv)) return GDN_ERR_UNSUPPORTED;
    if (E > kProjMaxK || (size_t)Hv * dv > (size_t)kProjMaxK) return GDN_ERR_UNSUPPORTED;
    if (dk % 16 != 0 || dv % 16 != 0) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

struct LayerWs {
    size_t x, z, y, g, beta, o, nsums, core, total;
};

// The prefill's own workspace first (so its header, the status word and the wait bound, is the
// layer workspace's), then x fp32 [T][conv_dim], z fp16 [T][Hv dv], the normalised output y
// bf16 [T][Hv dv], g and beta fp32 [T][Hv], the recurrence output fp32 [T][Hv dv] and the
// row-sum words of the norm formed in the prefill.  z is fp16, not bf16: a bf16 rounding of
// z, propagated through SiLU(z) and the output projection, took the layer output past its
// tolerance on some inputs (seven sequences of 1 key / 2 value heads: 1.17 of the bar with a
// bf16 z on the GPU and in a CPU emulation of the roundings; 0.78 with an fp16 or fp32 z).
LayerWs layer_ws(int T, int N, int Hk, int Hv, int dk, int dv) {
    const size_t C = 2 * (size_t)Hk * dk + (size_t)Hv * dv, Z = (size_t)Hv * dv;
    LayerWs w{};
    w.core = 0;
    w.x = w.core + align256(gdn::chunked_workspace_bytes(T, N, Hv, dk, dv));
    w.z = w.x + align256((size_t)T * C * 4);
    w.y = w.z + align256((size_t)T * Z * 2);
    w.g = w.y + align256((size_t)T * Z * 2);
    w.beta = w.g + align256((size_t)T * Hv * 4);
    w.o = w.beta + align256((size_t)T * Hv * 4);
    w.nsums = w.o + align256((size_t)T * Z * 4);
    w.total = w.nsums + align256(gdn::norm_epi_words(T, N, Hv, dv) * 8);
    return w;
}

// GDN_LAYER_NORM_SEPARATE set (and not "0"): the layer's prefill runs its gated RMSNorm as a
// pass of its own even where the prefill could form it (read at every call; for tests).
bool layer_norm_separate() {
    const char *v = std::getenv("GDN_LAYER_NORM_SEPARATE");
    return v && *v && std::strcmp(v, "0") != 0;
}

struct LayerDecodeWs {
    size_t x, z, g, beta, y, partial, total;
};

LayerDecodeWs layer_decode_ws(int B, int E, int Hk, int Hv, int dk, int dv) {
    const size_t C = 2 * (size_t)Hk * dk + (size_t)Hv * dv, Z = (size_t)Hv * dv;
    LayerDecodeWs w{};
    w.x = 0;
    w.z = w.x + align256((size_t)B * C * 4);
    w.g = w.z + align256((size_t)B * Z * 2);
    w.beta = w.g + align256((size_t)B * Hv * 4);
    w.y = w.beta + align256((size_t)B * Hv * 4);
    w.partial = w.y + align256((size_t)B * Z * 2);
    w.total = w.partial + align256((size_t)kDecodeProjSplits * B * E * 4);
    return w;
}

}  // namespace

int gdn_linear(const void *a, const void *w, void *y, int M, int N, int K, void *stream) {
    try {
        if (!proj_shape_ok(M, N, K)) return M < 0 || N <= 0 || K <= 0 ? GDN_ERR_BAD_SHAPE : GDN_ERR_UNSUPPORTED;
        if (!w || (M > 0 && (!a || !y))) return GDN_ERR_NULL_POINTER;
        if (!aligned16({a, w, y})) return GDN_ERR_ALIGN;
        const Range ra{a, (size_t)M * K * 2}, rw{w, (size_t)N * K * 2}, ry{y, (size_t)M * N * 2};
        if (overlap(ry, ra) || overlap(ry, rw)) return GDN_ERR_ALIAS;
        return linear_impl(a, w, y, M, N, K, (hipStream_t)stream);
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

int gdn_in_proj(const void *hidden, const void *w_in, void *x, void *z, float *g, float *beta, int T, int E,
                int Hk, int Hv, int dk, int dv, void *stream) {
    try {
        if (T < 0) return GDN_ERR_BAD_SHAPE;
        if (int e = check_layer_shape(E, Hk, Hv, dk, dv)) return e;
        if (!w_in || (T > 0 && (!hidden || !x || !z || !g || !beta))) return GDN_ERR_NULL_POINTER;
        if (!aligned16({hidden, w_in, x, z, g, beta})) return GDN_ERR_ALIGN;
        const size_t C = 2 * (size_t)Hk * dk + (size_t)Hv * dv, Z = (size_t)Hv * dv;
        const Range rh{hidden, (size_t)T * E * 2}, rw{w_in, (C + Z + 2 * (size_t)Hv) * E * 2},
            rx{x, (size_t)T * C * 2}, rz{z, (size_t)T * Z * 2}, rg{g, (size_t)T * Hv * 4}, rb{beta, rg.bytes};
        const Range outs[] = {rx, rz, rg, rb};
        for (int i = 0; i < 4; ++i) {
            if (overlap(outs[i], rh) || overlap(outs[i], rw)) return GDN_ERR_ALIAS;
            for (int j = i + 1; j < 4; ++j)
                if (overlap(outs[i], outs[j])) return GDN_ERR_ALIAS;
        }
        return in_proj_impl(hidden, w_in, x, z, g, beta, T, E, Hk, Hv, dk, dv, (hipStream_t)stream);
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

size_t gdn_layer_prefill_workspace_size(int T, int N, int Hk, int Hv, int dk, int dv) {
    if (T < 0 || N < 1 || N > kMaxSeqs || check_heads(Hk, Hv) != GDN_OK || !gdn::chunked_supported(dk, dv)) return 0;
    return layer_ws(T, N, Hk, Hv, dk, dv).total;
}

int gdn_layer_prefill(const void *hidden, const void *w_in, const void *conv_w, const void *gamma,
                      const void *w_out, const int32_t *cu_seqlens, int N, const void *conv_state_in,
                      void *conv_state_out, const float *initial_state, float *final_state, void *out, float scale,
                      float l2_eps, float norm_eps, int T, int E, int Hk, int Hv, int dk, int dv, int order,
                      void *workspace, size_t workspace_bytes, void *stream) {
    try {
        if (int e = check_seqs(cu_seqlens, N, T)) return e;
        if (int e = check_layer_shape(E, Hk, Hv, dk, dv)) return e;
        if (!gdn::chunked_supported(dk, dv) || !valid_order(order)) return GDN_ERR_UNSUPPORTED;
        if (!w_in || !conv_w || !gamma || !w_out || (T > 0 && (!hidden || !out))) return GDN_ERR_NULL_POINTER;
        if (!aligned16({hidden, w_in, conv_w, gamma, w_out, cu_seqlens, conv_state_in, conv_state_out,
                        initial_state, final_state, out, workspace}))
            return GDN_ERR_ALIGN;
        if (!std::isfinite(scale) || !(l2_eps >= 0.f) || !std::isfinite(l2_eps) || !(norm_eps >= 0.f) ||
            !std::isfinite(norm_eps))
            return GDN_ERR_BAD_SHAPE;
        const LayerWs L = layer_ws(T, N, Hk, Hv, dk, dv);
        if (!workspace || workspace_bytes < L.total) return GDN_ERR_WORKSPACE;
        const size_t C = 2 * (size_t)Hk * dk + (size_t)Hv * dv, Z = (size_t)Hv * dv;
        const size_t st_bytes = (size_t)N * Hv * dk * dv * 4, cs_bytes = (size_t)N * 3 * C * 4;
        const Range rh{hidden, (size_t)T * E * 2}, rwi{w_in, (C + Z + 2 * (size_t)Hv) * E * 2},
            rcw{conv_w, C * 4 * 2}, rgm{gamma, (size_t)dv * 2}, rwo{w_out, (size_t)E * Z * 2},
            rci{conv_state_in, cs_bytes}, rco{conv_state_out, cs_bytes}, rs0{initial_state, st_bytes},
            rsf{final_state, st_bytes}, rout{out, (size_t)T * E * 2}, rws{workspace, L.total};
        for (Range in : {rh, rwi, rcw, rgm, rwo, rci, rco, rs0, rsf, rout})
            if (overlap(rws, in)) return GDN_ERR_ALIAS;
        for (Range in : {rh, rwi, rcw, rgm, rwo, rci, rco, rs0, rsf})
            if (overlap(rout, in)) return GDN_ERR_ALIAS;
        for (Range in : {rh, rwi, rcw, rgm, rwo})
            if (overlap(rco, in) || overlap(rsf, in)) return GDN_ERR_ALIAS;
        // the output caches may replace the input ones exactly (and only exactly)
        if (overlap(rco, rs0) || overlap(rco, rsf) || bad_partial_alias(rco, rci) || bad_partial_alias(rsf, rs0) ||
            overlap(rsf, rci))
            return GDN_ERR_ALIAS;
        char *ws = static_cast<char *>(workspace);
        void *x = ws + L.x, *z = ws + L.z;
        float *g = reinterpret_cast<float *>(ws + L.g), *beta = reinterpret_cast<float *>(ws + L.beta);
        float *o = reinterpret_cast<float *>(ws + L.o);
        hipStream_t st = (hipStream_t)stream;
        if (int e = in_proj_impl(hidden, w_in, x, z, g, beta, T, E, Hk, Hv, dk, dv, st, true, true)) return e;
        // the normalised output y (bf16) feeds the output projection: formed by the prefill
        // where its schedule allows, else as a pass of its own over o
        void *y = ws + L.y;
        gdn::NormEpi ne{z, gamma, y, norm_eps, reinterpret_cast<unsigned long long *>(ws + L.nsums)};
        if (int e = prefill_impl(x, conv_w, cu_seqlens, N, conv_state_in, conv_state_out, g, beta, initial_state,
                                 final_state, o, scale, l2_eps, T, Hk, Hv, dk, dv, GDN_F32, order, ws + L.core,
                                 L.x - L.core, stream, 3, true, layer_norm_separate() ? nullptr : &ne))
            return e;
        gdn::NormArgs na{o, z, gamma, y, (long)T * Hv, dv, norm_eps, true};
        na.z_f16 = true;
        if (T > 0 && !ne.fused)
            if (int e = hip_status(gdn::launch_gated_rmsnorm(na, st))) return e;
        return linear_impl(y, w_out, out, T, E, (int)Z, st);
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

size_t gdn_layer_decode_workspace_size(int B, int E, int Hk, int Hv, int dk, int dv) {
    if (B < 0 || B > kMaxSeqs || E <= 0 || E > kProjMaxK || check_heads(Hk, Hv) != GDN_OK || dk <= 0 || dk > 256 ||
        dv <= 0 || dv > 256)
        return 0;
    return layer_decode_ws(B, E, Hk, Hv, dk, dv).total;
}

int gdn_layer_decode(const void *hidden, const void *w_in, const void *conv_w, const void *gamma,
                     const void *w_out, void *conv_state, float *state, void *out, float scale, float l2_eps,
                     float norm_eps, int B, int E, int Hk, int Hv, int dk, int dv, int order, void *workspace,
                     size_t workspace_bytes, void *stream) {
    try {
        if (B < 0 || B > kMaxSeqs) return GDN_ERR_BAD_SHAPE;
        if (int e = check_layer_shape(E, Hk, Hv, dk, dv)) return e;
        if (!pow2_in(dk, 16, 128) || !pow2_in(dv, 16, 128) || !valid_order(order)) return GDN_ERR_UNSUPPORTED;
        if (!w_in || !conv_w || !gamma || !w_out || (B > 0 && (!hidden || !conv_state || !state || !out)))
            return GDN_ERR_NULL_POINTER;
        if (!aligned16({hidden, w_in, conv_w, gamma, w_out, conv_state, state, out, workspace})) return GDN_ERR_ALIGN;
        if (!std::isfinite(scale) || !(l2_eps >= 0.f) || !std::isfinite(l2_eps) || !(norm_eps >= 0.f) ||
            !std::isfinite(norm_eps))
            return GDN_ERR_BAD_SHAPE;
        const LayerDecodeWs L = layer_decode_ws(B, E, Hk, Hv, dk, dv);
        if (!workspace || workspace_bytes < L.total) return GDN_ERR_WORKSPACE;
        const size_t C = 2 * (size_t)Hk * dk + (size_t)Hv * dv, Z = (size_t)Hv * dv;
        const Range rh{hidden, (size_t)B * E * 2}, rwi{w_in, (C + Z + 2 * (size_t)Hv) * E * 2},
            rcw{conv_w, C * 4 * 2}, rgm{gamma, (size_t)dv * 2}, rwo{w_out, (size_t)E * Z * 2},
            rcs{conv_state, (size_t)B * 3 * C * 4}, rst{state, (size_t)B * Hv * dk * dv * 4},
            rout{out, (size_t)B * E * 2}, rws{workspace, L.total};
        for (Range in : {rh, rwi, rcw, rgm, rwo, rcs, rst, rout})
            if (overlap(rws, in)) return GDN_ERR_ALIAS;
        for (Range in : {rh, rwi, rcw, rgm, rwo, rcs, rst})
            if (overlap(rout, in)) return GDN_ERR_ALIAS;
        for (Range in : {rh, rwi, rcw, rgm, rwo})
            if (overlap(rcs, in) || overlap(rst, in)) return GDN_ERR_ALIAS;
        if (overlap(rcs, rst)) return GDN_ERR_ALIAS;
        char *ws = static_cast<char *>(workspace);
        void *x = ws + L.x, *z = ws + L.z, *y = ws + L.y;
        float *g = reinterpret_cast<float *>(ws + L.g), *beta = reinterpret_cast<float *>(ws + L.beta);
        hipStream_t st = (hipStream_t)stream;
        if (int e = in_proj_impl(hidden, w_in, x, z, g, beta, B, E, Hk, Hv, dk, dv, st, true)) return e;
        if (B > 0) {
            // the decode step with the gated RMSNorm fused (x and the conv cache fp32, the
            // conv weights, z, gamma and the normalised output bf16)
            gdn::DecodeArgs a{x, conv_w, conv_state, g, beta, state, nullptr, scale, l2_eps, B, Hk, Hv, dk, dv,
                              false};
            a.order = order;
            a.z = z;
            a.gamma = gamma;
            a.out = y;
            a.norm_eps = norm_eps;
            a.layer_types = true;
            if (int e = hip_status(gdn::launch_decode(a, st))) return e;
        }
        return linear_impl(y, w_out, out, B, E, (int)Z, st, reinterpret_cast<float *>(ws + L.partial),
                           (size_t)kDecodeProjSplits * B * E);
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

}  // extern "C"

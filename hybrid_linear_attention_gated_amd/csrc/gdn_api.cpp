// gdn_api.cpp -- the extern "C" entry points declared in include/gdn.h:
// argument validation on the host (nothing is enqueued when it fails), pointer
// overlap checks, and dispatch to the kernels' launchers.
#include "gdn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <initializer_list>

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

int check_heads(int Hk, int Hv) {
    if (Hk <= 0 || Hv <= 0 || Hv % Hk != 0) return GDN_ERR_BAD_SHAPE;
    return GDN_OK;
}

int check_seqs(const int32_t *cu, int N, int T) {
    if (T < 0 || N < 1) return GDN_ERR_BAD_SHAPE;
    if (!cu && N != 1) return GDN_ERR_BAD_SHAPE;
    return GDN_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

bool valid_order(int order) { return order == GDN_ORDER_DECAY_FIRST || order == GDN_ORDER_RETRIEVE_FIRST; }

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
    (void)Hk;
    if (T < 0 || N < 1 || Hv <= 0) return 0;
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
        if (math != GDN_MATH_F32 && math != GDN_MATH_MFMA) return GDN_ERR_UNSUPPORTED;
        if (!valid_order(order)) return GDN_ERR_UNSUPPORTED;
        if (phases != 3 && math != GDN_MATH_MFMA) return GDN_ERR_UNSUPPORTED;
        if (!pow2_in(dk, 16, 128) || !pow2_in(dv, 16, 128)) return GDN_ERR_UNSUPPORTED;
        if (math == GDN_MATH_MFMA && !gdn::chunked_supported(dk, dv)) return GDN_ERR_UNSUPPORTED;
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
        return hip_status(chunked ? gdn::launch_prefill_chunked(a, st, phases) : gdn::launch_prefill_recurrent(a, st));
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
int prefill_impl(const void *x, const void *conv_w, const int32_t *cu_seqlens, int N, const void *conv_state_in,
                 void *conv_state_out, const float *g, const float *beta, const float *initial_state,
                 float *final_state, float *o, float scale, float l2_eps, int T, int Hk, int Hv, int dk, int dv,
                 int dtype, int order, void *workspace, size_t workspace_bytes, void *stream, int phases) {
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
        const size_t eb = elem_bytes(dtype);
        const size_t conv_dim = 2 * (size_t)Hk * dk + (size_t)Hv * dv;
        const size_t st_bytes = (size_t)N * Hv * dk * dv * 4;
        const Range rx{x, (size_t)T * conv_dim * eb}, rw{conv_w, conv_dim * 4 * eb};
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
        const gdn::FusedPrep fp{x, conv_w, conv_state_in, conv_state_out, dtype == GDN_BF16, l2_eps};
        gdn::PrefillArgs a{nullptr, nullptr, nullptr, g, beta, cu_seqlens, N, initial_state, final_state, o, scale,
                           T, Hk, Hv, dk, dv, workspace, workspace_bytes, &fp};
        a.order = order;
        return hip_status(gdn::launch_prefill_chunked(a, (hipStream_t)stream, phases));
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
        if (B < 0) return GDN_ERR_BAD_SHAPE;
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
        if (rows < 0) return GDN_ERR_BAD_SHAPE;
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

}  // extern "C"

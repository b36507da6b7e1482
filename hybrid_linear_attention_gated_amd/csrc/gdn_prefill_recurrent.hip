// gdn_prefill_recurrent.hip -- token-recurrent fp32 prefill of the gated delta
// rule over packed varlen sequences.
//
// Method: the recurrent-mode step of "Hugging Face Transformers: Qwen3.5-MoE
// series explained", section 4.3 (decay, retrieve, correct, write, read), one
// token at a time, all in fp32 arithmetic; with order = 1 the retrieval reads the
// state before the decay, as "7.6 Qwen3.5: the linear-attention hybrid" (section
// 7.6.2) writes the recurrence.  It serves GDN_MATH_F32 (whose
// 1e-4 RMS-relative accuracy leaves no room for 16-bit MFMA operands) and the
// head dims that the chunked MFMA path does not tile.
//
// Design: one workgroup per (sequence, value head); thread j owns state column
// j (dk fp32 registers).  Columns of the state evolve independently, so no
// reduction crosses threads; the token's k and q are broadcast through a
// double-buffered LDS slot, one barrier per token.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

template <int DK>
__global__ __launch_bounds__(128) void prefill_recurrent_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const int32_t *__restrict__ cu,
    const float *s0, float *sf, float *__restrict__ o, float scale, int Ttot, int Hk, int Hv, int dv, int order) {
    __shared__ float kq[2][2][DK];
    const int h = blockIdx.x, s = blockIdx.y;
    const int j = threadIdx.x;
    const bool act = j < dv;
    const int kh = h / (Hv / Hk);
    const int t0 = seq_begin(cu, s), t1 = seq_end(cu, s, Ttot);

    float S[DK];
    const size_t st_off = ((size_t)s * Hv + h) * DK * dv;
#pragma unroll
    for (int i = 0; i < DK; ++i) S[i] = (s0 && act) ? s0[st_off + (size_t)i * dv + j] : 0.f;

    for (int t = t0; t < t1; ++t) {
        const int buf = (t - t0) & 1;
        for (int i = threadIdx.x; i < DK; i += blockDim.x) {
            kq[buf][0][i] = k[((size_t)t * Hk + kh) * DK + i];
            kq[buf][1][i] = scale * q[((size_t)t * Hk + kh) * DK + i];
        }
        __syncthreads();
        const float a = __expf(g[(size_t)t * Hv + h]);
        const float b = beta[(size_t)t * Hv + h];
        if (act) {
            float m = 0.f;
            if (order == 0) {
#pragma unroll
                for (int i = 0; i < DK; ++i) { S[i] *= a; m = fmaf(S[i], kq[buf][0][i], m); }
            } else {
#pragma unroll
                for (int i = 0; i < DK; ++i) { m = fmaf(S[i], kq[buf][0][i], m); S[i] *= a; }
            }
            const float d = b * (v[((size_t)t * Hv + h) * dv + j] - m);
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < DK; ++i) { S[i] = fmaf(kq[buf][0][i], d, S[i]); acc = fmaf(S[i], kq[buf][1][i], acc); }
            o[((size_t)t * Hv + h) * dv + j] = acc;
        }
    }
    if (sf && act) {
#pragma unroll
        for (int i = 0; i < DK; ++i) sf[st_off + (size_t)i * dv + j] = S[i];
    }
}

template <int DK>
static hipError_t launch_rec_t(const PrefillArgs &a, hipStream_t st) {
    const int threads = a.dv <= 64 ? 64 : 128;
    hipLaunchKernelGGL((prefill_recurrent_kernel<DK>), dim3(a.Hv, a.N), dim3(threads), 0, st, a.q, a.k, a.v, a.g,
                       a.beta, a.cu, a.s0, a.sf, a.o, a.scale, a.T, a.Hk, a.Hv, a.dv, a.order);
    return hipGetLastError();
}

hipError_t launch_prefill_recurrent(const PrefillArgs &a, hipStream_t st) {
    switch (a.dk) {
        case 16: return launch_rec_t<16>(a, st);
        case 32: return launch_rec_t<32>(a, st);
        case 64: return launch_rec_t<64>(a, st);
        case 128: return launch_rec_t<128>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn

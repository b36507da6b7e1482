// gdn_prep.hip -- fused depthwise causal conv1d (kernel 4) + SiLU + split +
// per-head L2 normalisation of q and k, for packed varlen sequences.
//
// Method: "7.6 Qwen3.5: the linear-attention hybrid" (LLM full-stack book),
// section 7.6.2 -- conv over conv_dim = 2*key_dim + value_dim channels with one
// filter per channel and left context only, then L2-normalised q and k; the conv
// cache (last inputs of each sequence) follows "Hugging Face Transformers:
// Qwen3.5-MoE series explained", section 8.2.
//
// Design (HBM-streaming, ~6 flop per element): each lane owns 8 consecutive
// channels (one 16-byte load per token for bf16 x), a wave covers 512 channels
// and walks 16 consecutive tokens, keeping the 3-token conv window in
// registers, so x is read once (plus a 3-row warm-up per wave that hits L2) and
// the fp32 q/k/v are written once with 16-byte stores.  The L2 norm of a head of dk channels is a
// reduction over dk/8 aligned lanes (xor shuffles), with no LDS and no barrier.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int kPrepTokPerWave = 16;
constexpr int kPrepWaves = 4;
constexpr int kPrepChan = 8 * kWave;  // channels per wave

template <typename T, int DK>
__global__ __launch_bounds__(kPrepWaves * kWave) void prep_kernel(
    const T *__restrict__ x, const T *__restrict__ w, const int32_t *__restrict__ cu, int N,
    const T *__restrict__ cs_in, float *__restrict__ q, float *__restrict__ k, float *__restrict__ v,
    int Ttot, int Hk, int Hv, int dv, int conv_dim, float eps) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int c0 = blockIdx.x * kPrepChan + lane * 8;
    const bool active = c0 < conv_dim;
    const int qk_dim = Hk * DK;
    const int t_begin = (blockIdx.y * kPrepWaves + wave) * kPrepTokPerWave;
    if (t_begin >= Ttot) return;  // whole wave exits together
    const int t_end = min(t_begin + kPrepTokPerWave, Ttot);

    float wt[4][8];
    if (active) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // conv_w[c][0..3]: 4 taps of one channel are contiguous
#pragma unroll
            for (int j = 0; j < 4; ++j) wt[j][i] = to_f32(w[(size_t)(c0 + i) * kConvK + j]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) wt[j][i] = 0.f;
    }

    // where this lane's 8 channels go (fp32 outputs)
    float *dst;
    size_t dst_row;
    bool normed;
    if (c0 < qk_dim) { dst = q; dst_row = (size_t)qk_dim; normed = true; }
    else if (c0 < 2 * qk_dim) { dst = k; dst_row = (size_t)qk_dim; normed = true; }
    else { dst = v; dst_row = (size_t)Hv * dv; normed = false; }
    const int dst_col = c0 < qk_dim ? c0 : (c0 < 2 * qk_dim ? c0 - qk_dim : c0 - 2 * qk_dim);

    int s = find_seq(cu, N, t_begin);
    int ts = seq_begin(cu, s), te = seq_end(cu, s, Ttot);

    // window h[0] oldest .. h[2] newest: inputs at t-3, t-2, t-1
    float h[3][8];
    auto fill_window = [&](int t) {
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int pos = t - 3 + j;
            if (!active) {
#pragma unroll
                for (int i = 0; i < 8; ++i) h[j][i] = 0.f;
            } else if (pos >= ts) {
                Vec8<T>::load(x + (size_t)pos * conv_dim + c0, h[j]);
            } else if (cs_in) {
                Vec8<T>::load(cs_in + ((size_t)s * kConvHist + (kConvHist + (pos - ts))) * conv_dim + c0, h[j]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) h[j][i] = 0.f;
            }
        }
    };
    fill_window(t_begin);

    for (int t = t_begin; t < t_end; ++t) {
        if (t >= te) {  // entered the next non-empty sequence: restart the history
            while (seq_end(cu, s, Ttot) <= t) ++s;
            ts = seq_begin(cu, s);
            te = seq_end(cu, s, Ttot);
            fill_window(t);
        }
        float xt[8], y[8];
        if (active) Vec8<T>::load(x + (size_t)t * conv_dim + c0, xt);
        else {
#pragma unroll
            for (int i = 0; i < 8; ++i) xt[i] = 0.f;
        }
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float acc = wt[0][i] * h[0][i];
            acc = fmaf(wt[1][i], h[1][i], acc);
            acc = fmaf(wt[2][i], h[2][i], acc);
            acc = fmaf(wt[3][i], xt[i], acc);
            y[i] = silu(acc);
            ss = fmaf(y[i], y[i], ss);
        }
        ss = group_sum<DK / 8>(ss);
        if (normed) {
            const float r = rsqrtf(ss + eps);
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] *= r;
        }
        if (active) Vec8<float>::store(dst + (size_t)t * dst_row + dst_col, y);
#pragma unroll
        for (int i = 0; i < 8; ++i) { h[0][i] = h[1][i]; h[1][i] = h[2][i]; h[2][i] = xt[i]; }
    }
}

// conv_state_out[s] = the last three inputs of sequence s (from conv_state_in
// when the sequence is shorter than three).  One thread per (s, channel); it
// reads all three slots before writing, so conv_state_out may alias conv_state_in.
template <typename T>
__global__ __launch_bounds__(256) void conv_state_out_kernel(
    const T *__restrict__ x, const int32_t *__restrict__ cu, int N, const T *cs_in, T *cs_out,
    int Ttot, int conv_dim) {
    const int c = blockIdx.x * blockDim.x + threadIdx.x;
    const int s = blockIdx.y;
    if (c >= conv_dim || s >= N) return;
    const int ts = seq_begin(cu, s);
    const int L = seq_end(cu, s, Ttot) - ts;
    float vals[kConvHist];
#pragma unroll
    for (int j = 0; j < kConvHist; ++j) {
        const int pos = L - kConvHist + j;
        if (pos >= 0) vals[j] = to_f32(x[(size_t)(ts + pos) * conv_dim + c]);
        else if (cs_in) vals[j] = to_f32(cs_in[((size_t)s * kConvHist + (kConvHist + pos)) * conv_dim + c]);
        else vals[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < kConvHist; ++j) cs_out[((size_t)s * kConvHist + j) * conv_dim + c] = from_f32<T>(vals[j]);
}

template <typename T, int DK>
static hipError_t launch_prep_t(const PrepArgs &a, hipStream_t st) {
    const int conv_dim = 2 * a.Hk * a.dk + a.Hv * a.dv;
    if (a.T > 0) {
        dim3 grid((conv_dim + kPrepChan - 1) / kPrepChan,
                  (a.T + kPrepWaves * kPrepTokPerWave - 1) / (kPrepWaves * kPrepTokPerWave));
        hipLaunchKernelGGL((prep_kernel<T, DK>), grid, dim3(kPrepWaves * kWave), 0, st,
                           (const T *)a.x, (const T *)a.w, a.cu, a.N, (const T *)a.cs_in,
                           a.q, a.k, a.v, a.T, a.Hk, a.Hv, a.dv, conv_dim, a.eps);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.cs_out) {
        dim3 grid((conv_dim + 255) / 256, a.N);
        hipLaunchKernelGGL((conv_state_out_kernel<T>), grid, dim3(256), 0, st,
                           (const T *)a.x, a.cu, a.N, (const T *)a.cs_in, (T *)a.cs_out, a.T, conv_dim);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <typename T>
static hipError_t launch_prep_dk(const PrepArgs &a, hipStream_t st) {
    switch (a.dk) {
        case 16: return launch_prep_t<T, 16>(a, st);
        case 32: return launch_prep_t<T, 32>(a, st);
        case 64: return launch_prep_t<T, 64>(a, st);
        case 128: return launch_prep_t<T, 128>(a, st);
        case 256: return launch_prep_t<T, 256>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prep(const PrepArgs &a, hipStream_t st) {
    return a.bf16 ? launch_prep_dk<bf16>(a, st) : launch_prep_dk<float>(a, st);
}

}  // namespace gdn

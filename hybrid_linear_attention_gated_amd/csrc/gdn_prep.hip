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
// and 16 consecutive tokens.  A wave issues the loads of all 19 rows it needs
// (its 16 tokens and the 3 before them) before it computes anything, so every
// wave keeps ~19 KB in flight; the 3-token conv window then slides through
// registers, each row converted once.  The fp32 q/k/v are written once with
// 16-byte stores.  The L2 norm of a head of dk channels is a reduction over
// dk/8 aligned lanes (xor shuffles), with no LDS and no barrier.  Sequence
// starts inside a wave's range take a uniform slow path that reads the conv
// cache (or zeros) for the first three tokens.
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int kPrepTokPerWave = 16;
constexpr int kPrepWaves = 4;
constexpr int kPrepChan = 8 * kWave;  // channels per wave

// conv_state_out[s] = the last three inputs of sequence s (from conv_state_in when the
// sequence is shorter than three), for channels c of this thread.
template <typename T>
__device__ __forceinline__ void conv_state_out_channel(const T *__restrict__ x, const int32_t *__restrict__ cu,
                                                       int s, const T *cs_in, T *cs_out, int Ttot, int conv_dim,
                                                       int c) {
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

// Blocks with blockIdx.y < ty_blocks run the conv; when cs_out_fused is set (the
// output cache does not alias the input cache), blocks ty_blocks .. ty_blocks + N - 1
// write conv_state_out for sequence blockIdx.y - ty_blocks.
template <typename T, int DK>
__global__ __launch_bounds__(kPrepWaves * kWave) void prep_kernel(
    const T *__restrict__ x, const T *__restrict__ w, const int32_t *__restrict__ cu, int N,
    const T *__restrict__ cs_in, T *__restrict__ cs_out_fused, float *__restrict__ q, float *__restrict__ k,
    float *__restrict__ v, int Ttot, int Hk, int Hv, int dv, int conv_dim, float eps, int ty_blocks) {
    if ((int)blockIdx.y >= ty_blocks) {
        const int s = blockIdx.y - ty_blocks;
        for (int c = blockIdx.x * (kPrepWaves * kWave) + threadIdx.x; c < conv_dim;
             c += gridDim.x * (kPrepWaves * kWave))
            conv_state_out_channel<T>(x, cu, s, cs_in, cs_out_fused, Ttot, conv_dim, c);
        return;
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int c0 = blockIdx.x * kPrepChan + lane * 8;
    const bool active = c0 < conv_dim;
    const int cc = active ? c0 : 0;   // in-bounds channel for inactive lanes (their results are dropped)
    const int qk_dim = Hk * DK;
    const int t_begin = (blockIdx.y * kPrepWaves + wave) * kPrepTokPerWave;
    if (t_begin >= Ttot) return;  // whole wave exits together
    const int nt = min(kPrepTokPerWave, Ttot - t_begin);

    // rows t_begin - 3 .. t_begin + 15, clamped into [0, Ttot - 1]; rows outside the
    // current sequence are replaced below
    constexpr int NR = kPrepTokPerWave + kConvHist;
    Raw8<T> rows[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int pos = min(max(t_begin - kConvHist + r, 0), Ttot - 1);
        rows[r].load(x + (size_t)pos * conv_dim + cc);
    }

    float wt[4][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        // conv_w[c][0..3]: 4 taps of one channel are contiguous
#pragma unroll
        for (int j = 0; j < 4; ++j) wt[j][i] = to_f32(w[(size_t)(cc + i) * kConvK + j]);
    }

    // where this lane's 8 channels go (fp32 outputs)
    float *dst;
    size_t dst_row;
    bool normed;
    if (c0 < qk_dim) { dst = q; dst_row = (size_t)qk_dim; normed = true; }
    else if (c0 < 2 * qk_dim) { dst = k; dst_row = (size_t)qk_dim; normed = true; }
    else { dst = v; dst_row = (size_t)Hv * dv; normed = false; }
    const int dst_col = c0 < qk_dim ? c0 : (c0 < 2 * qk_dim ? c0 - qk_dim : c0 - 2 * qk_dim);

    // sequence bounds are wave-uniform: keep them in scalar registers so the boundary
    // tests below are scalar branches
    int s = __builtin_amdgcn_readfirstlane(find_seq(cu, N, t_begin));
    int ts = __builtin_amdgcn_readfirstlane(seq_begin(cu, s));
    int te = __builtin_amdgcn_readfirstlane(seq_end(cu, s, Ttot));

    // window h[0] oldest .. h[2] newest: inputs at t-3, t-2, t-1
    float h[3][8];
#pragma unroll
    for (int j = 0; j < 3; ++j) rows[j].to_f32(h[j]);
    float *dp = dst + (size_t)t_begin * dst_row + dst_col;
    // SIMPLE: the 16 tokens and the 3 before them lie in one sequence and every lane is
    // active -- no per-token tests at all (every wave of a long sequence but its first)
    auto run = [&](auto simple_tag) __attribute__((always_inline)) {
        constexpr bool SIMPLE = decltype(simple_tag)::value;
        constexpr bool FULL = SIMPLE;
#pragma unroll
        for (int i = 0; i < kPrepTokPerWave; ++i) {
            const int t = t_begin + i;
            const bool live = FULL || i < nt;
            if (!SIMPLE && live && t >= te) {   // a new (non-empty) sequence starts at t
                while (seq_end(cu, s, Ttot) <= t) ++s;
                s = __builtin_amdgcn_readfirstlane(s);
                ts = __builtin_amdgcn_readfirstlane(seq_begin(cu, s));
                te = __builtin_amdgcn_readfirstlane(seq_end(cu, s, Ttot));
            }
            if (!SIMPLE && live && t - kConvHist < ts) {   // window reaches before the sequence start
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    const int pos = t - kConvHist + j;
                    if (pos < ts) {
                        if (cs_in && active) {
                            Raw8<T> c;
                            c.load(cs_in + ((size_t)s * kConvHist + (kConvHist + (pos - ts))) * conv_dim + cc);
                            c.to_f32(h[j]);
                        } else {
#pragma unroll
                            for (int e = 0; e < 8; ++e) h[j][e] = 0.f;
                        }
                    }
                }
            }
            float xt[8], y[8];
            rows[i + kConvHist].to_f32(xt);
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float acc = wt[0][e] * h[0][e];
                acc = fmaf(wt[1][e], h[1][e], acc);
                acc = fmaf(wt[2][e], h[2][e], acc);
                acc = fmaf(wt[3][e], xt[e], acc);
                y[e] = silu(acc);
                ss = fmaf(y[e], y[e], ss);
            }
            ss = group_sum<DK / 8>(ss);
            if (normed) {
                const float r = rsqrtf(ss + eps);
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] *= r;
            }
            if (FULL || (active && live)) Vec8<float>::store(dp, y);
            dp += dst_row;
#pragma unroll
            for (int e = 0; e < 8; ++e) { h[0][e] = h[1][e]; h[1][e] = h[2][e]; h[2][e] = xt[e]; }
        }
    };
    const bool simple = nt == kPrepTokPerWave && (int)(blockIdx.x + 1) * kPrepChan <= conv_dim &&
                        t_begin - kConvHist >= ts && t_begin + kPrepTokPerWave <= te;
    if (simple) run(std::true_type{});
    else run(std::false_type{});
}

// Standalone conv_state_out pass for the case where the output cache aliases the
// input cache: one thread per (s, channel); it reads all three slots before
// writing, and it runs after the conv has read the input cache.
template <typename T>
__global__ __launch_bounds__(256) void conv_state_out_kernel(
    const T *__restrict__ x, const int32_t *__restrict__ cu, int N, const T *cs_in, T *cs_out,
    int Ttot, int conv_dim) {
    const int c = blockIdx.x * blockDim.x + threadIdx.x;
    const int s = blockIdx.y;
    if (c >= conv_dim || s >= N) return;
    conv_state_out_channel<T>(x, cu, s, cs_in, cs_out, Ttot, conv_dim, c);
}

template <typename T, int DK>
static hipError_t launch_prep_t(const PrepArgs &a, hipStream_t st) {
    const int conv_dim = 2 * a.Hk * a.dk + a.Hv * a.dv;
    // the cache copy joins the conv launch unless it overwrites the cache the conv reads
    const bool fuse_cs = a.cs_out && !(a.cs_in && a.cs_in == a.cs_out);
    const int ty = (a.T + kPrepWaves * kPrepTokPerWave - 1) / (kPrepWaves * kPrepTokPerWave);
    const int gy = ty + (fuse_cs ? a.N : 0);
    if (gy > 0) {
        dim3 grid((conv_dim + kPrepChan - 1) / kPrepChan, gy);
        hipLaunchKernelGGL((prep_kernel<T, DK>), grid, dim3(kPrepWaves * kWave), 0, st,
                           (const T *)a.x, (const T *)a.w, a.cu, a.N, (const T *)a.cs_in,
                           fuse_cs ? (T *)a.cs_out : (T *)nullptr, a.q, a.k, a.v, a.T, a.Hk, a.Hv, a.dv,
                           conv_dim, a.eps, ty);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.cs_out && !fuse_cs) {
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

template <typename T>
static hipError_t launch_cs_out_t(const PrepArgs &a, hipStream_t st) {
    const int conv_dim = 2 * a.Hk * a.dk + a.Hv * a.dv;
    if (!a.cs_out || a.N <= 0) return hipSuccess;
    dim3 grid((conv_dim + 255) / 256, a.N);
    hipLaunchKernelGGL((conv_state_out_kernel<T>), grid, dim3(256), 0, st,
                       (const T *)a.x, a.cu, a.N, (const T *)a.cs_in, (T *)a.cs_out, a.T, conv_dim);
    return hipGetLastError();
}

hipError_t launch_conv_state_out(const PrepArgs &a, hipStream_t st) {
    return a.bf16 ? launch_cs_out_t<bf16>(a, st) : launch_cs_out_t<float>(a, st);
}

hipError_t launch_prep(const PrepArgs &a, hipStream_t st) {
    return a.bf16 ? launch_prep_dk<bf16>(a, st) : launch_prep_dk<float>(a, st);
}

}  // namespace gdn

// gdn_decode.hip -- one decode step of the Gated DeltaNet mixer for B sequences:
// conv-cache advance + conv + SiLU + L2(q, k) + one step of the gated delta rule
// on the fp32 state, in place.
//
// Method: the decode branch of "Hugging Face Transformers: Qwen3.5-MoE series
// explained", section 8.2 (conv-cache update, then the recurrent rule, then
// both caches written back) with the recurrent-mode step of section 4.3:
// S <- a S; m = S^T k; delta = b (v - m); S <- S + k delta^T; o = S^T q
// (order 1: m is taken from the state before the decay, the recurrence as "7.6 Qwen3.5:
// the linear-attention hybrid", section 7.6.2, writes it).
//
// Design (HBM-bound, ~0.84 flop per byte): one 256-thread workgroup per
// (sequence, key head) owns the conv channels of that key head and of all value
// heads that read it, so the in-place conv-cache shift has a single writer per
// channel.  For each value head the dk x dv fp32 state is streamed once: thread
// (row group, column quad) keeps its rows as float4 registers, so a wave reads
// and writes whole 512-byte rows.  Since S' = a S + k delta^T, both reductions
// needed (S^T k and S^T q, over dk) are taken from the OLD state in the same
// pass:  m = a (S^T k) (order 1: S^T k),  o = a (S^T q) + delta (k . q).  Row-group partial sums
// are combined with xor shuffles inside a wave and through LDS across waves.
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int kDecThreads = 256;

template <typename T, typename TW>
__device__ __forceinline__ float conv_step(const T *__restrict__ x, const TW *__restrict__ w, T *cs,
                                           int b, int c, int conv_dim) {
    // window = [slot0, slot1, slot2, x]; afterwards the cache is [slot1, slot2, x]
    T *cb = cs + (size_t)b * kConvHist * conv_dim + c;
    const float s0 = to_f32(cb[0]);
    const float s1 = to_f32(cb[(size_t)conv_dim]);
    const T s2raw = cb[2 * (size_t)conv_dim];
    const T xraw = x[(size_t)b * conv_dim + c];
    const float s2 = to_f32(s2raw), xn = to_f32(xraw);
    const TW *wc = w + (size_t)c * kConvK;
    float acc = to_f32(wc[0]) * s0;
    acc = fmaf(to_f32(wc[1]), s1, acc);
    acc = fmaf(to_f32(wc[2]), s2, acc);
    acc = fmaf(to_f32(wc[3]), xn, acc);
    cb[0] = cb[(size_t)conv_dim];
    cb[(size_t)conv_dim] = s2raw;
    cb[2 * (size_t)conv_dim] = xraw;
    return silu(acc);
}

// Four consecutive elements of the element type as one vector access (8 or 16 bytes).
__device__ __forceinline__ void load4(const bf16 *p, float *o) {
    const bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (float)v[e];
}
__device__ __forceinline__ void load4(const float *p, float *o) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = v[e];
}
__device__ __forceinline__ void store4(bf16 *p, const float *i) {
    bf16x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (bf16)i[e];
    *reinterpret_cast<bf16x4 *>(p) = v;
}
__device__ __forceinline__ void store4(float *p, const float *i) {
    *reinterpret_cast<f32x4 *>(p) = f32x4{i[0], i[1], i[2], i[3]};
}

// GATED: the output row of each value head goes through the gated RMSNorm epilogue
// ("7.6 Qwen3.5: the linear-attention hybrid", sections 7.6.2 and 7.6.3) before it is
// stored: out = o * rsqrt(mean o^2 + norm_eps) * gamma * SiLU(z), in the gate's element
// type TG.  The dv outputs of a head sit in the first dv/4 lanes of wave 0 (4 each), so the
// mean square is one reduction inside that lane group.
// T: element type of x and the conv cache; TW: of the conv weights.
template <typename T, typename TW, typename TG, int DK, int DV, bool GATED>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void decode_kernel(
    const T *__restrict__ x, const TW *__restrict__ w, T *cs, const float *__restrict__ g,
    const float *__restrict__ beta, float *state, float *__restrict__ o, float scale, float eps,
    int Hk, int Hv, const TG *__restrict__ z, const TG *__restrict__ gamma, TG *__restrict__ out, float norm_eps,
    int order) {
    constexpr int TPR = DV / 4;                  // threads per state row (one float4 each)
    constexpr int RG = kDecThreads / TPR;        // row groups
    constexpr int RPT = DK >= RG ? DK / RG : 1;  // rows per thread
    constexpr int NW = kDecThreads / kWave;
    static_assert(TPR <= kWave, "row must fit in a wave");

    __shared__ float qk_s[2 * DK];   // raw SiLU(conv) of q then k
    // 16-byte aligned: the cross-wave sums and v are moved as one float4 per lane (16 lanes
    // cover 256 contiguous bytes, one LDS cycle without bank conflicts)
    __shared__ __attribute__((aligned(16))) float v_s[DV];
    __shared__ __attribute__((aligned(16))) float red[NW][2][DV];
    __shared__ float scal[3];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int b = blockIdx.x / Hk, kh = blockIdx.x % Hk;
    const int group = Hv / Hk;
    const int conv_dim = 2 * Hk * DK + Hv * DV;
    const int cg = tid % TPR, rg = tid / TPR;
    const bool row_active = rg < DK;

    // first value head's state: issue the loads before the conv work
    float4 S[RPT];
    auto load_state = [&](int h) {
        const float *sp = state + ((size_t)b * Hv + h) * DK * DV + 4 * cg;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int i = rg + RG * r;
            // non-temporal: the state is read once per step and is as large as the Infinity
            // Cache, so its lines are not kept there (they would evict, for example, a
            // prefill workspace that the next prefill call rewrites and reads back)
            S[r] = make_float4(0, 0, 0, 0);
            if (row_active) {
                const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(sp + (size_t)i * DV));
                S[r] = make_float4(t[0], t[1], t[2], t[3]);
            }
        }
    };
    load_state(kh * group);
    // gated epilogue: this lane's gate and gain values, loaded with the state (lanes 0 ..
    // TPR - 1 of wave 0 hold a head's outputs), so the store at the end does not wait for them
    float zf[4] = {0.f, 0.f, 0.f, 0.f}, gf[4] = {0.f, 0.f, 0.f, 0.f};
    const bool gate_lane = GATED && wave == 0 && rg == 0;
    auto load_gate = [&](int h) {
        if (gate_lane) load4(z + ((size_t)b * Hv + h) * DV + 4 * cg, zf);
    };
    if (gate_lane) load4(gamma + 4 * cg, gf);
    load_gate(kh * group);

    // q and k channels of this key head
    for (int ch = tid; ch < 2 * DK; ch += kDecThreads) {
        const int c = ch < DK ? kh * DK + ch : Hk * DK + kh * DK + (ch - DK);
        qk_s[ch] = conv_step(x, w, cs, b, c, conv_dim);
    }
    __syncthreads();
    if (wave < 3) {
        float acc = 0.f;
        for (int i = lane; i < DK; i += kWave) {
            const float qi = qk_s[i], ki = qk_s[DK + i];
            acc += wave == 0 ? qi * qi : (wave == 1 ? ki * ki : qi * ki);
        }
        acc = group_sum<kWave>(acc);
        if (lane == 0) scal[wave] = acc;
    }
    __syncthreads();
    const float rq = rsqrtf(scal[0] + eps) * scale;  // q_hat * scale
    const float rk = rsqrtf(scal[1] + eps);
    const float kq = scal[2] * rq * rk;                // k_hat . (scale q_hat)

    // the scaled key and query entries of this thread's rows, read from LDS where they are used
    // (the lanes of a row group read the same word: broadcast reads) instead of held in 2 RPT
    // registers: with them the kernel needed 150 VGPRs, three workgroups per compute unit and
    // 5.3 rounds of workgroups at decode256; now four per compute unit, four rounds (decode
    // step 1-3 us faster by HIP events in the bench's order, same arithmetic)
    auto kr = [&](int r) { return row_active ? qk_s[DK + rg + RG * r] * rk : 0.f; };
    auto qr = [&](int r) { return row_active ? qk_s[rg + RG * r] * rq : 0.f; };

    for (int gi = 0; gi < group; ++gi) {
        const int h = kh * group + gi;
        if (gi > 0) {
            load_state(h);
            load_gate(h);
        }
        for (int ch = tid; ch < DV; ch += kDecThreads)
            v_s[ch] = conv_step(x, w, cs, b, 2 * Hk * DK + h * DV + ch, conv_dim);

        float pm[4] = {0, 0, 0, 0}, pq[4] = {0, 0, 0, 0};
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            pm[0] = fmaf(S[r].x, kr(r), pm[0]); pm[1] = fmaf(S[r].y, kr(r), pm[1]);
            pm[2] = fmaf(S[r].z, kr(r), pm[2]); pm[3] = fmaf(S[r].w, kr(r), pm[3]);
            pq[0] = fmaf(S[r].x, qr(r), pq[0]); pq[1] = fmaf(S[r].y, qr(r), pq[1]);
            pq[2] = fmaf(S[r].z, qr(r), pq[2]); pq[3] = fmaf(S[r].w, qr(r), pq[3]);
        }
#pragma unroll
        for (int m = TPR; m < kWave; m <<= 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pm[e] += __shfl_xor(pm[e], m, kWave);
                pq[e] += __shfl_xor(pq[e], m, kWave);
            }
        }
        if (lane < TPR) {
            *reinterpret_cast<f32x4 *>(&red[wave][0][4 * cg]) = f32x4{pm[0], pm[1], pm[2], pm[3]};
            *reinterpret_cast<f32x4 *>(&red[wave][1][4 * cg]) = f32x4{pq[0], pq[1], pq[2], pq[3]};
        }
        __syncthreads();   // red and v_s complete
        const float a = __expf(g[(size_t)b * Hv + h]);
        const float bt = beta[(size_t)b * Hv + h];
        f32x4 sk = zero4(), sq = zero4();
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            sk += *reinterpret_cast<const f32x4 *>(&red[ww][0][4 * cg]);
            sq += *reinterpret_cast<const f32x4 *>(&red[ww][1][4 * cg]);
        }
        const f32x4 v4 = *reinterpret_cast<const f32x4 *>(&v_s[4 * cg]);
        float delta[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            delta[e] = bt * (v4[e] - (order == 0 ? a * sk[e] : sk[e]));
            pq[e] = a * sq[e] + delta[e] * kq;   // output column 4cg+e
        }
        if constexpr (GATED) {
            if (wave == 0) {   // rg == 0 is lanes 0 .. TPR - 1 of wave 0
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) ss = fmaf(pq[e], pq[e], ss);
                ss = group_sum<TPR>(ss);
                const float rn = rsqrtf(ss * (1.0f / DV) + norm_eps);
                if (rg == 0) {
                    float r4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) r4[e] = pq[e] * rn * gf[e] * silu(zf[e]);
                    store4(out + ((size_t)b * Hv + h) * DV + 4 * cg, r4);
                }
            }
        } else if (rg == 0) {
            *reinterpret_cast<float4 *>(o + ((size_t)b * Hv + h) * DV + 4 * cg) = make_float4(pq[0], pq[1], pq[2], pq[3]);
        }
        if (row_active) {
            float *sp = state + ((size_t)b * Hv + h) * DK * DV + 4 * cg;
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const int i = rg + RG * r;
                float4 n;
                n.x = fmaf(a, S[r].x, kr(r) * delta[0]);
                n.y = fmaf(a, S[r].y, kr(r) * delta[1]);
                n.z = fmaf(a, S[r].z, kr(r) * delta[2]);
                n.w = fmaf(a, S[r].w, kr(r) * delta[3]);
                *reinterpret_cast<float4 *>(sp + (size_t)i * DV) = n;
            }
        }
        __syncthreads();   // red / v_s reused by the next value head
    }
}

template <typename T, typename TW, typename TG, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t st) {
    if (a.B == 0) return hipSuccess;
    if (a.out) {
        hipLaunchKernelGGL((decode_kernel<T, TW, TG, DK, DV, true>), dim3(a.B * a.Hk), dim3(kDecThreads), 0, st,
                           (const T *)a.x, (const TW *)a.w, (T *)a.cs, a.g, a.beta, a.state, (float *)nullptr,
                           a.scale, a.eps, a.Hk, a.Hv, (const TG *)a.z, (const TG *)a.gamma, (TG *)a.out,
                           a.norm_eps, a.order);
    } else if constexpr (std::is_same<T, TW>::value && std::is_same<T, TG>::value) {
        hipLaunchKernelGGL((decode_kernel<T, T, T, DK, DV, false>), dim3(a.B * a.Hk), dim3(kDecThreads), 0, st,
                           (const T *)a.x, (const T *)a.w, (T *)a.cs, a.g, a.beta, a.state, a.o, a.scale, a.eps,
                           a.Hk, a.Hv, (const T *)nullptr, (const T *)nullptr, (T *)nullptr, 0.f, a.order);
    } else {
        return hipErrorInvalidValue;   // mixed element types only with the gated output
    }
    return hipGetLastError();
}

template <typename T, typename TW, typename TG, int DK>
static hipError_t launch_decode_dv(const DecodeArgs &a, hipStream_t st) {
    switch (a.dv) {
        case 16: return launch_decode_t<T, TW, TG, DK, 16>(a, st);
        case 32: return launch_decode_t<T, TW, TG, DK, 32>(a, st);
        case 64: return launch_decode_t<T, TW, TG, DK, 64>(a, st);
        case 128: return launch_decode_t<T, TW, TG, DK, 128>(a, st);
        default: return hipErrorInvalidValue;
    }
}

template <typename T, typename TW, typename TG>
static hipError_t launch_decode_dk(const DecodeArgs &a, hipStream_t st) {
    switch (a.dk) {
        case 16: return launch_decode_dv<T, TW, TG, 16>(a, st);
        case 32: return launch_decode_dv<T, TW, TG, 32>(a, st);
        case 64: return launch_decode_dv<T, TW, TG, 64>(a, st);
        case 128: return launch_decode_dv<T, TW, TG, 128>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t st) {
    if (a.layer_types) return launch_decode_dk<float, bf16, bf16>(a, st);   // the layer's decode
    return a.bf16 ? launch_decode_dk<bf16, bf16, bf16>(a, st) : launch_decode_dk<float, float, float>(a, st);
}

}  // namespace gdn

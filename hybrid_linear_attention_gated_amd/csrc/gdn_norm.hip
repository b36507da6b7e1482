// gdn_norm.hip -- gated RMSNorm epilogue of the linear-attention output:
//   out[r][j] = y[r][j] * rsqrt(mean_j y[r][j]^2 + eps) * gamma[j] * SiLU(z[r][j])
// over rows r = (token, value head) of dv channels ("7.6 Qwen3.5: the
// linear-attention hybrid", section 7.6.2: the layer output passes a gated
// RMSNorm, o = RMSNorm(y) * SiLU(z) with z a separate projection of the input;
// the RMSNorm is that of section 7.6.3, computed in fp32, with the per-channel
// gain passed as applied).
//
// Design (HBM-bound: 4 + 2 e bytes per element for element size e, no reuse):
// a lane owns 4 consecutive channels of a row (one float4 of y, 4 elements of z
// and of the output); min(64, dv/4) lanes form a row, so a wave covers one or
// more whole rows and the sum of squares is a DPP / xor reduction inside the
// lane group.  dv = 256 takes two float4 per lane.  The gain is read once per
// lane and kept in registers.  y and z are read once, with non-temporal loads:
// after kernels that leave the Infinity Cache full of written lines, allocating
// them there costs a write-back per line (layer_4k rows, 67 MB: 17 us instead of
// 25 us; 16 us vs 15 us when the cache holds no written lines).
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int kNormThreads = 256;

// Four elements as fp32: loads are non-temporal (data read once), stores plain.
template <typename T> struct Vec4;
template <> struct Vec4<float> {
    static __device__ __forceinline__ void load(const float *p, float *o) {
        const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
        o[0] = v[0]; o[1] = v[1]; o[2] = v[2]; o[3] = v[3];
    }
    static __device__ __forceinline__ void store(float *p, const float *i) {
        *reinterpret_cast<f32x4 *>(p) = f32x4{i[0], i[1], i[2], i[3]};
    }
};
template <> struct Vec4<f16> {
    static __device__ __forceinline__ void load(const f16 *p, float *o) {
        const f16x4 v = __builtin_nontemporal_load(reinterpret_cast<const f16x4 *>(p));
        o[0] = (float)v[0]; o[1] = (float)v[1]; o[2] = (float)v[2]; o[3] = (float)v[3];
    }
};
template <> struct Vec4<bf16> {
    static __device__ __forceinline__ void load(const bf16 *p, float *o) {
        const bf16x4 v = __builtin_nontemporal_load(reinterpret_cast<const bf16x4 *>(p));
        o[0] = (float)v[0]; o[1] = (float)v[1]; o[2] = (float)v[2]; o[3] = (float)v[3];
    }
    static __device__ __forceinline__ void store(bf16 *p, const float *i) {
        bf16x4 v;
        v[0] = (bf16)i[0]; v[1] = (bf16)i[1]; v[2] = (bf16)i[2]; v[3] = (bf16)i[3];
        *reinterpret_cast<bf16x4 *>(p) = v;
    }
};

template <int DV>
struct NormShape {
    static constexpr int LPR = DV / 4 < kWave ? DV / 4 : kWave;   // lanes per row
    static constexpr int NV = DV / (4 * LPR);                      // float4 per lane and row
    static constexpr int RPT = 4;                                  // rows per lane group
    static constexpr int RPB = kNormThreads / LPR * RPT;           // rows per workgroup
};

// Each lane group takes RPT rows spaced kNormThreads / LPR apart and issues all their
// loads (RPT * NV of y and as many of z per lane) before any arithmetic.
template <typename TZ, typename T, int DV>
__global__ __launch_bounds__(kNormThreads) void gated_rmsnorm_kernel(
    const float *y, const TZ *z, const T *__restrict__ gamma, T *out, long rows, float eps) {
    using S = NormShape<DV>;
    constexpr int LPR = S::LPR, NV = S::NV, RPT = S::RPT, STRIDE = kNormThreads / LPR;
    const int tid = threadIdx.x, sub = tid % LPR;
    const long r0 = (long)blockIdx.x * S::RPB + tid / LPR;
    float gm[NV][4], yv[RPT][NV][4], zv[RPT][NV][4];
#pragma unroll
    for (int i = 0; i < NV; ++i) Vec4<T>::load(gamma + 4 * (sub + LPR * i), gm[i]);
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        const long r = r0 + (long)k * STRIDE;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c = 4 * (sub + LPR * i);
            if (r < rows) {
                Vec4<float>::load(y + r * DV + c, yv[k][i]);
                Vec4<TZ>::load(z + r * DV + c, zv[k][i]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) { yv[k][i][e] = 0.f; zv[k][i][e] = 0.f; }
            }
        }
    }
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        const long r = r0 + (long)k * STRIDE;
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) ss = fmaf(yv[k][i][e], yv[k][i][e], ss);
        ss = group_sum<LPR>(ss);
        const float rn = rsqrtf(ss * (1.0f / DV) + eps);
        if (r < rows) {
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                float o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = yv[k][i][e] * rn * gm[i][e] * silu(zv[k][i][e]);
                Vec4<T>::store(out + r * DV + 4 * (sub + LPR * i), o);
            }
        }
    }
}

template <typename TZ, typename T, int DV>
static hipError_t launch_norm_t(const NormArgs &a, hipStream_t st) {
    constexpr int RPB = NormShape<DV>::RPB;
    const long blocks = (a.rows + RPB - 1) / RPB;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gated_rmsnorm_kernel<TZ, T, DV>), dim3((unsigned)blocks), dim3(kNormThreads), 0, st, a.y,
                       (const TZ *)a.z, (const T *)a.gamma, (T *)a.out, a.rows, a.eps);
    return hipGetLastError();
}

template <typename TZ, typename T>
static hipError_t launch_norm_dv(const NormArgs &a, hipStream_t st) {
    switch (a.dv) {
        case 16: return launch_norm_t<TZ, T, 16>(a, st);
        case 32: return launch_norm_t<TZ, T, 32>(a, st);
        case 64: return launch_norm_t<TZ, T, 64>(a, st);
        case 128: return launch_norm_t<TZ, T, 128>(a, st);
        case 256: return launch_norm_t<TZ, T, 256>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gated_rmsnorm(const NormArgs &a, hipStream_t st) {
    if (a.bf16 && a.z_f16) return launch_norm_dv<f16, bf16>(a, st);   // the layer prefill's fp16 gate
    return a.bf16 ? launch_norm_dv<bf16, bf16>(a, st) : launch_norm_dv<float, float>(a, st);
}

}  // namespace gdn

// gdn_chunk_f32.hip -- the chunked (chunk 64, WY / UT) form of the gated delta rule in
// fp32 arithmetic for small heads (dk, dv in {16, 32, 64}), the GDN_MATH_F32_CHUNKED
// arithmetic of gdn_chunk_prefill.
//
// Method: the recurrent-mode step of "Hugging Face Transformers: Qwen3.5-MoE series
// explained", section 4.3 (decay, retrieve, correct, write, read), unrolled over a chunk of
// c <= 64 tokens exactly as the MFMA path does (key-major state S[dk][dv], local cumulative
// log-decay G_t = g_1 + ... + g_t, retrieval-side decay Gr = G, or G - g when the retrieval
// reads the state before the decay as "7.6 Qwen3.5: the linear-attention hybrid", section
// 7.6.2, writes it):
//
//   A[t][i] = b_t e^{Gr_t - G_i} (k_t . k_i)  (i < t),   T = (I + A)^-1 (forward substitution)
//   W = T diag(b e^{Gr}) K,   U = T diag(b) V,   Delta = U - W S
//   O[t] = scale (e^{G_t} q_t S + sum_{i <= t} e^{G_t - G_i} (q_t . k_i) Delta[i])
//   S' = e^{G_c} S + sum_i e^{G_c - G_i} k_i Delta[i]^T
//
// Every product is an fp32 sum on the vector ALU; nothing is rounded below fp32.
//
// Design: one 256-thread workgroup per (sequence, value head) carries the state in LDS
// across the sequence's chunks (the sequential dependence); per chunk, each product is a
// dot-product loop over LDS with threads spread over its output elements.  The triangular
// solve gives each of 64 threads one column of T in registers (T is unit lower triangular:
// row t needs only rows i < t of the same column).  This path serves the small head sizes
// and the fp32 accuracy bar (1e-4 RMS); the 128-wide heads of the model shapes use the MFMA
// path.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int kF32Threads = 256;

template <int DK, int DV>
struct F32Smem {
    static constexpr int KLD = DK + 1, VLD = DV + 1, CLD = kChunk + 1;   // padded row strides (floats)
    static constexpr int K = 0;                         // keys        [64][KLD]
    static constexpr int Q = K + kChunk * KLD;          // queries     [64][KLD] (times scale)
    static constexpr int V = Q + kChunk * KLD;          // values      [64][VLD], then U, then Delta
    static constexpr int W = V + kChunk * VLD;          // W           [64][KLD]
    static constexpr int U = W + kChunk * KLD;          // U           [64][VLD]
    static constexpr int A = U + kChunk * VLD;          // A, then T   [64][CLD]
    static constexpr int P = A + kChunk * CLD;          // P           [64][CLD]
    static constexpr int S = P + kChunk * CLD;          // state       [DK][DV]
    static constexpr int G = S + DK * DV;               // G, Gr, beta, beta e^Gr, e^{G_c - G} [5][64]
    static constexpr int SIZE = (G + 5 * kChunk) * 4;   // bytes
    static_assert(SIZE <= 160 * 1024, "LDS");
};

template <int DK, int DV>
__global__ __launch_bounds__(kF32Threads) void chunk_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const int32_t *__restrict__ cu, int Ttot,
    int Hk, int Hv, float scale, const float *s0, float *sf, float *__restrict__ o, int order) {
    using SM = F32Smem<DK, DV>;
    __shared__ float smem[SM::SIZE / 4];
    float *Ks = smem + SM::K, *Qs = smem + SM::Q, *Vs = smem + SM::V, *Ws = smem + SM::W, *Us = smem + SM::U;
    float *As = smem + SM::A, *Ps = smem + SM::P, *Ss = smem + SM::S;
    float *Gs = smem + SM::G, *GRs = Gs + kChunk, *Bs = Gs + 2 * kChunk, *BEG = Gs + 3 * kChunk, *DC = Gs + 4 * kChunk;
    constexpr int KLD = SM::KLD, VLD = SM::VLD, CLD = SM::CLD;

    const int s = blockIdx.x / Hv, h = blockIdx.x % Hv, kh = h / (Hv / Hk);
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int t0s = seq_begin(cu, s), L = seq_end(cu, s, Ttot) - t0s;
    const size_t st_off = ((size_t)s * Hv + h) * DK * DV;

    for (int e = tid; e < DK * DV; e += kF32Threads) Ss[e] = s0 ? s0[st_off + e] : 0.f;

    for (int c0 = 0; c0 < L; c0 += kChunk) {
        const int n = min(kChunk, L - c0);
        const int tb = t0s + c0;
        __syncthreads();   // the previous chunk is done with every buffer
        // ---- the chunk's keys, queries (times scale), values and gates; rows >= n are zero
        for (int e = tid; e < kChunk * DK; e += kF32Threads) {
            const int t = e / DK, d = e % DK;
            const bool live = t < n;
            const size_t at = ((size_t)(tb + (live ? t : 0)) * Hk + kh) * DK + d;
            Ks[t * KLD + d] = live ? k[at] : 0.f;
            Qs[t * KLD + d] = live ? scale * q[at] : 0.f;
        }
        for (int e = tid; e < kChunk * DV; e += kF32Threads) {
            const int t = e / DV, j = e % DV;
            Vs[t * VLD + j] = t < n ? v[((size_t)(tb + t) * Hv + h) * DV + j] : 0.f;
        }
        if (wave == 0) {
            const bool live = lane < n;
            const float gg = live ? g[(size_t)(tb + lane) * Hv + h] : 0.f;
            float G = gg;   // inclusive prefix sum over the chunk
            for (int m = 1; m < kWave; m <<= 1) {
                const float y = __shfl_up(G, m, kWave);
                if (lane >= m) G += y;
            }
            const float Gr = order == 0 ? G : G - gg;
            const float bb = live ? beta[(size_t)(tb + lane) * Hv + h] : 0.f;
            Gs[lane] = G;
            GRs[lane] = Gr;
            Bs[lane] = bb;
            BEG[lane] = bb * expf(Gr);
            DC[lane] = expf(__shfl(G, kWave - 1, kWave) - G);
        }
        __syncthreads();
        // ---- A (strictly lower) and P (lower with diagonal)
        for (int e = tid; e < kChunk * kChunk; e += kF32Threads) {
            const int t = e / kChunk, i = e % kChunk;
            float kk = 0.f, qk = 0.f;
            if (i <= t) {
                for (int d = 0; d < DK; ++d) {
                    const float ki = Ks[i * KLD + d];
                    kk = fmaf(Ks[t * KLD + d], ki, kk);
                    qk = fmaf(Qs[t * KLD + d], ki, qk);
                }
            }
            As[t * CLD + i] = i < t ? Bs[t] * expf(GRs[t] - Gs[i]) * kk : 0.f;
            Ps[t * CLD + i] = i <= t ? expf(Gs[t] - Gs[i]) * qk : 0.f;
        }
        __syncthreads();
        // ---- T = (I + A)^-1 by forward substitution: thread j keeps column j of T in
        // registers; row t of T is e_t - sum_{i < t} A[t][i] T[i] (A is read, T replaces it
        // row by row after every thread has read row t of A)
        if (tid < kChunk) {
            const int j = tid;
            float col[kChunk];
#pragma unroll
            for (int t = 0; t < kChunk; ++t) {
                float x = t == j ? 1.f : 0.f;
#pragma unroll
                for (int i = 0; i < t; ++i) x = fmaf(-As[t * CLD + i], col[i], x);
                col[t] = x;
            }
            // one wave: every lane's reads of A above precede these writes in program order
#pragma unroll
            for (int t = 0; t < kChunk; ++t) As[t * CLD + j] = col[t];
        }
        __syncthreads();
        // ---- W = T diag(b e^{Gr}) K and U = T diag(b) V
        for (int e = tid; e < kChunk * (DK + DV); e += kF32Threads) {
            const int t = e / (DK + DV), r = e % (DK + DV);
            float acc = 0.f;
            if (r < DK) {
                for (int i = 0; i <= t; ++i) acc = fmaf(As[t * CLD + i] * BEG[i], Ks[i * KLD + r], acc);
                Ws[t * KLD + r] = acc;
            } else {
                const int j = r - DK;
                for (int i = 0; i <= t; ++i) acc = fmaf(As[t * CLD + i] * Bs[i], Vs[i * VLD + j], acc);
                Us[t * VLD + j] = acc;
            }
        }
        __syncthreads();
        // ---- Delta = U - W S (into the value buffer)
        for (int e = tid; e < kChunk * DV; e += kF32Threads) {
            const int t = e / DV, j = e % DV;
            float acc = Us[t * VLD + j];
            for (int d = 0; d < DK; ++d) acc = fmaf(-Ws[t * KLD + d], Ss[d * DV + j], acc);
            Vs[t * VLD + j] = acc;
        }
        __syncthreads();
        // ---- outputs from the state before the chunk: O = e^G Q S + P Delta
        for (int e = tid; e < n * DV; e += kF32Threads) {
            const int t = e / DV, j = e % DV;
            float qs = 0.f, pd = 0.f;
            for (int d = 0; d < DK; ++d) qs = fmaf(Qs[t * KLD + d], Ss[d * DV + j], qs);
            for (int i = 0; i <= t; ++i) pd = fmaf(Ps[t * CLD + i], Vs[i * VLD + j], pd);
            o[((size_t)(tb + t) * Hv + h) * DV + j] = fmaf(expf(Gs[t]), qs, pd);
        }
        __syncthreads();
        // ---- S' = e^{G_c} S + sum_i e^{G_c - G_i} k_i Delta_i^T
        const float eGc = expf(Gs[kChunk - 1]);
        for (int e = tid; e < DK * DV; e += kF32Threads) {
            const int d = e / DV, j = e % DV;
            float acc = 0.f;
            for (int i = 0; i < n; ++i) acc = fmaf(DC[i] * Ks[i * KLD + d], Vs[i * VLD + j], acc);
            Ss[e] = fmaf(eGc, Ss[e], acc);
        }
    }
    __syncthreads();
    if (sf)
        for (int e = tid; e < DK * DV; e += kF32Threads) sf[st_off + e] = Ss[e];
}

bool chunked_f32_supported(int dk, int dv) {
    return (dk == 16 || dk == 32 || dk == 64) && (dv == 16 || dv == 32 || dv == 64);
}

template <int DK, int DV>
static hipError_t launch_f32_t(const PrefillArgs &a, hipStream_t st) {
    const int units = a.N * a.Hv;
    if (units <= 0) return hipSuccess;
    hipLaunchKernelGGL((chunk_f32_kernel<DK, DV>), dim3(units), dim3(kF32Threads), 0, st, a.q, a.k, a.v, a.g,
                       a.beta, a.cu, a.T, a.Hk, a.Hv, a.scale, a.s0, a.sf, a.o, a.order);
    return hipGetLastError();
}

template <int DK>
static hipError_t launch_f32_dv(const PrefillArgs &a, hipStream_t st) {
    switch (a.dv) {
        case 16: return launch_f32_t<DK, 16>(a, st);
        case 32: return launch_f32_t<DK, 32>(a, st);
        case 64: return launch_f32_t<DK, 64>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prefill_chunked_f32(const PrefillArgs &a, hipStream_t st) {
    switch (a.dk) {
        case 16: return launch_f32_dv<16>(a, st);
        case 32: return launch_f32_dv<32>(a, st);
        case 64: return launch_f32_dv<64>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn

// gdn_device.hpp -- device-side helpers shared by the gfx950 kernels:
// element conversion, wavefront reductions, MFMA fragment types and the
// sequence/chunk bookkeeping for packed varlen batches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kConvK = 4;          // conv kernel width
constexpr int kConvHist = kConvK - 1;
constexpr int kChunk = 64;         // chunk length of the chunked prefill

// ---------------------------------------------------------------- element I/O

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// gfx950 converts with round-to-nearest-even (v_cvt_pk_bf16_f32)
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Load / store 8 consecutive elements as fp32.
template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
    static __device__ __forceinline__ void load(const bf16 *p, float *out) {
        bf16x8 v = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = (float)v[i];
    }
    static __device__ __forceinline__ void store(bf16 *p, const float *in) {
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (bf16)in[i];
        *reinterpret_cast<bf16x8 *>(p) = v;
    }
};
template <> struct Vec8<float> {
    static __device__ __forceinline__ void load(const float *p, float *out) {
        float4 a = *reinterpret_cast<const float4 *>(p);
        float4 b = *reinterpret_cast<const float4 *>(p + 4);
        out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
        out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
    }
    static __device__ __forceinline__ void store(float *p, const float *in) {
        *reinterpret_cast<float4 *>(p) = make_float4(in[0], in[1], in[2], in[3]);
        *reinterpret_cast<float4 *>(p + 4) = make_float4(in[4], in[5], in[6], in[7]);
    }
};

template <typename T> struct Raw8;    // 8 elements as loaded, converted later
template <> struct Raw8<bf16> {
    bf16x8 v;
    __device__ __forceinline__ void load(const bf16 *p) { v = *reinterpret_cast<const bf16x8 *>(p); }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (bf16)0.f;
    }
    __device__ __forceinline__ void to_f32(float *o) const {
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = (float)v[i];
    }
};
template <> struct Raw8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float *p) {
        a = *reinterpret_cast<const float4 *>(p);
        b = *reinterpret_cast<const float4 *>(p + 4);
    }
    __device__ __forceinline__ void zero() { a = make_float4(0.f, 0.f, 0.f, 0.f); b = a; }
    __device__ __forceinline__ void to_f32(float *o) const {
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
};


// SiLU y * sigmoid(y) with the hardware reciprocal (about 1 ulp) instead of an
// IEEE division sequence; for y < -88 the exponential overflows to +inf and the
// result is -0, the limit of the function.
__device__ __forceinline__ float silu(float y) { return y * __builtin_amdgcn_rcpf(1.0f + __expf(-y)); }

// ---------------------------------------------------------------- reductions

// Sum over aligned groups of `width` lanes (width a power of two <= 64).  Within a
// 16-lane row the steps are DPP moves (no LDS): quad permutes [1,0,3,2] and
// [2,3,0,1] sum each quad, the half-row mirror adds the other quad of each 8 and the
// row mirror the other half of the row; wider groups continue with xor shuffles.
template <int ctrl>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), ctrl, 0xF, 0xF, false));
}
template <int width>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (width >= 2) v += dpp_mov<0xB1>(v);    // quad_perm(1, 0, 3, 2)
    if constexpr (width >= 4) v += dpp_mov<0x4E>(v);    // quad_perm(2, 3, 0, 1)
    if constexpr (width >= 8) v += dpp_mov<0x141>(v);   // row_half_mirror
    if constexpr (width >= 16) v += dpp_mov<0x140>(v);  // row_mirror
#pragma unroll
    for (int m = 16; m < width; m <<= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// ---------------------------------------------------------------- varlen bookkeeping

__device__ __forceinline__ int seq_begin(const int32_t *cu, int s) { return cu ? cu[s] : 0; }
__device__ __forceinline__ int seq_end(const int32_t *cu, int s, int T) { return cu ? cu[s + 1] : T; }

// Sequence index containing token t (largest s with cu[s] <= t); cu[N] = T.
__device__ __forceinline__ int find_seq(const int32_t *cu, int N, int t) {
    if (!cu) return 0;
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ int n_chunks(int len) { return (len + kChunk - 1) / kChunk; }

// Index of the first chunk of sequence s in the packed chunk list (chunks
// restart at every sequence start).  O(s) scan; N is small on this path.
__device__ __forceinline__ int chunk_base(const int32_t *cu, int s) {
    if (!cu) return 0;
    int base = 0;
    for (int i = 0; i < s; ++i) base += n_chunks(cu[i + 1] - cu[i]);
    return base;
}

// ---------------------------------------------------------------- MFMA

// D += A * B with A 16x32, B 32x16 (bf16), D 16x16 (fp32).  Lane l holds
// A[l%16][k(l/16, v)], B[k(l/16, v)][l%16] for v < 8 and D[4*(l/16)+r][l%16].
// Any bijection k(kg, v) onto 0..31 that A and B share gives the same product.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Two-term bf16 representation of an fp32 value: hi = bf16(x), lo = bf16(x - hi)
// (about 16 significant bits together).  A product of two split operands is
// taken as hi*hi + hi*lo + lo*hi on bf16 MFMA.
struct Split8 {
    bf16x8 hi, lo;
};
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// hi / lo of two values as packed bf16 pairs: one paired conversion gives both hi, whose
// fp32 values are the pair's high halves moved up (shift) or masked in place, then one
// paired conversion of the two remainders.  Same result as converting each value alone.
__device__ __forceinline__ void split_pair(float x0, float x1, unsigned &hi, unsigned &lo) {
    hi = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{x0, x1}, bf16x2));
    const float h0 = __builtin_bit_cast(float, hi << 16), h1 = __builtin_bit_cast(float, hi & 0xffff0000u);
    lo = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{x0 - h0, x1 - h1}, bf16x2));
}
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ Split8 split8(const float *x) {
    unsigned h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split_pair(x[2 * i], x[2 * i + 1], h[i], l[i]);
    return Split8{__builtin_bit_cast(bf16x8, u32x4v{h[0], h[1], h[2], h[3]}),
                  __builtin_bit_cast(bf16x8, u32x4v{l[0], l[1], l[2], l[3]})};
}
// hi / lo of four values as packed bf16 quads
__device__ __forceinline__ void split4(const float *x, bf16x4 *hi, bf16x4 *lo) {
    unsigned h[2], l[2];
    split_pair(x[0], x[1], h[0], l[0]);
    split_pair(x[2], x[3], h[1], l[1]);
    *hi = __builtin_bit_cast(bf16x4, u32x2{h[0], h[1]});
    *lo = __builtin_bit_cast(bf16x4, u32x2{l[0], l[1]});
}
__device__ __forceinline__ f32x4 mfma16x3(const Split8 &a, const Split8 &b, f32x4 c) {
    c = mfma16(a.lo, b.hi, c);
    c = mfma16(a.hi, b.lo, c);
    return mfma16(a.hi, b.hi, c);
}
// The three partial products in separate accumulators: three independent MFMA chains
// that issue back to back instead of one chain whose every step waits for the last.
struct Acc3 {
    f32x4 hh, hl, lh;
};
__device__ __forceinline__ Acc3 acc3_zero() {
    const f32x4 z{0.f, 0.f, 0.f, 0.f};
    return Acc3{z, z, z};
}
__device__ __forceinline__ void mfma3_acc(Acc3 &s, const Split8 &a, const Split8 &b) {
    s.lh = mfma16(a.lo, b.hi, s.lh);
    s.hl = mfma16(a.hi, b.lo, s.hl);
    s.hh = mfma16(a.hi, b.hi, s.hh);
}
__device__ __forceinline__ f32x4 acc3_sum(const Acc3 &s) { return s.hh + (s.hl + s.lh); }
// a * b from zero with the three products independent
__device__ __forceinline__ f32x4 mfma16x3p(const Split8 &a, const Split8 &b) {
    Acc3 s = acc3_zero();
    mfma3_acc(s, a, b);
    return acc3_sum(s);
}

// The k order used when a B operand is built from two fp32 D tiles held in
// registers (rows 0-15 in tile 0, rows 16-31 in tile 1): lane group kg holds
// k = 4kg..4kg+3 (tile 0) and 16+4kg..16+4kg+3 (tile 1).  Every A operand that
// meets such a B uses the same order.
__device__ __forceinline__ int kperm(int kg, int v) { return (v < 4) ? (4 * kg + v) : (16 + 4 * kg + (v - 4)); }

// Gather the 8 B-operand values of two stacked accumulator tiles (see kperm).
__device__ __forceinline__ void gather8(f32x4 t0, f32x4 t1, float *x) {
    x[0] = t0[0]; x[1] = t0[1]; x[2] = t0[2]; x[3] = t0[3];
    x[4] = t1[0]; x[5] = t1[1]; x[6] = t1[2]; x[7] = t1[3];
}
__device__ __forceinline__ f16x8 pack_h(f32x4 t0, f32x4 t1) {
    f16x8 r;
    r[0] = (f16)t0[0]; r[1] = (f16)t0[1]; r[2] = (f16)t0[2]; r[3] = (f16)t0[3];
    r[4] = (f16)t1[0]; r[5] = (f16)t1[1]; r[6] = (f16)t1[2]; r[7] = (f16)t1[3];
    return r;
}
__device__ __forceinline__ Split8 split_tiles(f32x4 t0, f32x4 t1) {
    float x[8];
    gather8(t0, t1, x);
    return split8(x);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace gdn

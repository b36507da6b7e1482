// gdn_chunk.hip -- chunked (chunk 64, WY / UT form) prefill of the gated delta
// rule on MFMA for gfx950, for packed varlen sequences with initial and final
// states.
//
// Method.  The recurrence is the recurrent-mode GatedDeltaNet step of "Hugging
// Face Transformers: Qwen3.5-MoE series explained", section 4.3; its prefill
// is the chunk-mode call of section 8.2, which returns the outputs and the last
// state.  The chunk form below follows from unrolling that recurrence over a
// chunk of c <= 64 tokens (key-major state S[dk][dv], local cumulative
// log-decay G_t = g_1 + ... + g_t; the query scale multiplies the outputs, see below):
//
//   A[t][i] = b_t e^{G_t - G_i} (k_t . k_i)  for i < t,   T = (I + A)^-1
//   W = T diag(b e^G) K,     U = T diag(b) V,      Delta = U - W S
//   P[t][i] = e^{G_t - G_i} (q_t . k_i)  for i <= t
//   O = diag(e^G) Q S + P Delta = Qt S + Ol,   Qt = diag(e^G) Q - P W,  Ol = P U
//   S' = e^{G_c} S + K^T diag(e^{G_c - G}) Delta
//
// It equals the token recurrence in exact arithmetic (the CPU tests check the
// fp64 version of it against the token-by-token oracle).  With order = 1 the
// retrieval reads the state before the decay, as "7.6 Qwen3.5: the linear-attention
// hybrid" (section 7.6.2) writes the recurrence; unrolling it puts Gr_t = G_t - g_t
// in place of G_t in the first factor of A and in W (Gr = G for order 0), and
// leaves U, P, O and S' as they are.
//
// Precision.  Inputs q, k, v are fp32.  The outputs of this layer are heavy
// tailed (the largest |o| is tens of times its RMS), so one bf16 rounding of
// an operand costs up to ~2^-9 of the largest value, which is more than the
// 2e-2 RMS-relative accuracy the layer is held to.  Products therefore use
//  - in the chunk-local kernel: two-term bf16 splits (hi + lo) of both operands,
//    three MFMAs per product (K K^T, K Q^T, the block solves, and the four
//    products that form W', Qt, U', Ol);
//  - in the state pass: fp16 MFMA (11-bit significand) with W', Qt and the
//    state as single fp16 operands, and K and Delta' as bf16 hi + lo pairs
//    (three MFMAs for K^T Delta'); U' and Ol enter the fp32 accumulators with a
//    relative step of 2^-16 (24-bit floats, as precise as a hi + lo pair).
//    The query scale is applied to the fp32 outputs after the MFMAs (O is linear in
//    it), so it never enters a 16-bit operand.  fp16 operands assume |state| < 6.5e4;
//    the fp32 master state is never rounded, and a state beyond that range makes the
//    outputs non-finite, which the state pass reports in the workspace status word.
//
// Kernels.
//  chunk_local_kernel: the (chunk, value head) items are independent; the kernel is
//    persistent, one workgroup per compute unit looping over its head's chunks
//    (FUSED: it also runs the conv + SiLU + L2 prep of its chunk's tokens from x).
//    Explicit T = (I + A)^-1 and M = P T by block back substitution, then four
//    products.  Writes -W' = -diag(e^{G_c - G}) W and Qt as fp16 MFMA A-operand
//    fragments, K^T as bf16 hi / lo A-operand fragments, and
//    U' = diag(e^{G_c - G}) U and Ol^T as accumulator-layout tiles of 24-bit floats
//    (fp32 with the low byte rounded away, 12 bytes per lane and tile), so the
//    state pass reads every operand with one coalesced load per lane and every
//    product accumulates straight into its MFMA chain:
//      Delta' = diag(e^{G_c - G}) Delta = U' + (-W') S,   O^T = Ol^T + S^T Qt^T,
//      S' = e^{G_c} S + K^T Delta'.
//    O is formed transposed (the same fragments with A and B swapped) so that a
//    lane holds 4 consecutive columns of an output row: one 16-byte store per tile.
//  state_pass_kernel: one workgroup per (sequence, value head, two 16-column
//    strips of the state); a strip's fp32 state lives in MFMA accumulators for
//    the whole sequence and the chunk loop runs the three lines above, with the
//    chunk's A operands double-buffered in LDS by two copy waves.
//    Accumulator tiles are reused as B operands directly: the k index of an
//    MFMA may be permuted as long as A and B share the permutation, and the
//    stored A fragments carry the permutation that matches two stacked
//    accumulator tiles (kperm).
//
// Schedules (host side, end of file): the two kernels run one after the other, or
// in segments whose chunk-local and state-pass phases overlap on two streams, or
// concurrently, the state pass waiting for each record's ready flag while the
// chunk-local kernel, on the other compute units, publishes them.  In the layer's
// prefill at D = 128 the concurrent schedule's state pass also forms the gated RMSNorm
// of the outputs (norm_waves): o stays in LDS and only the normalised rows are stored.
#include <algorithm>
#include <mutex>
#include <numeric>
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

// Byte offsets inside one (chunk, value head) workspace record.
template <int D>
struct Rec {
    static constexpr int NKS = D / 32;                  // 32-wide k steps over the head dim
    static constexpr int NTD = D / 16;                  // 16-wide tiles over the head dim
    static constexpr int W_OFF = 0;                     // -W' f16 A frags [4 row tiles][NKS][64 lanes][8]
    static constexpr int Q_OFF = W_OFF + 64 * D * 2;    // Qt  f16 A frags [4][NKS][64][8]
    static constexpr int K_OFF = Q_OFF + 64 * D * 2;    // K^T bf16 A frags, hi and lo: [2][NTD row tiles][2][64][8]
    static constexpr int U_OFF = K_OFF + 64 * D * 4;    // U'  24-bit tiles [NTD col tiles][4 row tiles][64][12 B]
                                                        //   (W' = diag(e^{G_c - G_t}) W, U' likewise)
    static constexpr int O_OFF = U_OFF + 64 * D * 3;    // Ol^T 24-bit tiles [NTD][4][64][12 B] (rows = value column)
    static constexpr int GM_OFF = O_OFF + 64 * D * 3;   // e^{G_c}, f32, stored 4 times; then the query scale
    static constexpr int SIZE = GM_OFF + 256;           // padded to a multiple of 256 bytes
};

// Wave-parallel: first chunk index of sequence s in the packed chunk list.
__device__ __forceinline__ int chunk_base_wave(const int32_t *cu, int s) {
    const int lane = threadIdx.x & (kWave - 1);
    int acc = 0;
    if (cu) {
        for (int i0 = 0; i0 < s; i0 += kWave) {
            const int i = i0 + lane;
            if (i < s) acc += n_chunks(cu[i + 1] - cu[i]);
        }
    }
    for (int m = 1; m < kWave; m <<= 1) acc += __shfl_xor(acc, m, kWave);
    return acc;
}

// Wave-parallel: which sequence holds packed chunk gc, which chunk of it, and the
// sequence's token range [sb_out, se_out) (from the same loads).  Returns false when gc is
// past the last chunk.
__device__ __forceinline__ bool locate_chunk_wave(const int32_t *cu, int N, int Ttot, int gc, int &s_out,
                                                  int &c_out, int &sb_out, int &se_out) {
    const int lane = threadIdx.x & (kWave - 1);
    if (!cu) {
        s_out = 0; c_out = gc; sb_out = 0; se_out = Ttot;
        return gc < n_chunks(Ttot);
    }
    int base = 0;
    for (int i0 = 0; i0 < N; i0 += kWave) {
        const int i = i0 + lane;
        const int ta = i < N ? cu[i] : 0, tb = i < N ? cu[i + 1] : 0;
        const int n = i < N ? n_chunks(tb - ta) : 0;
        int incl = n;
        for (int o = 1; o < kWave; o <<= 1) {
            const int y = __shfl_up(incl, o, kWave);
            if (lane >= o) incl += y;
        }
        const int excl = base + incl - n;
        const unsigned long long hit = __ballot(i < N && n > 0 && gc >= excl && gc < excl + n);
        if (hit) {
            const int src = __ffsll((long long)hit) - 1;
            s_out = i0 + src;
            c_out = gc - __shfl(excl, src, kWave);
            sb_out = __builtin_amdgcn_readfirstlane(__shfl(ta, src, kWave));
            se_out = __builtin_amdgcn_readfirstlane(__shfl(tb, src, kWave));
            return true;
        }
        base += __shfl(incl, kWave - 1, kWave);
    }
    return false;
}

// Buffer resource over `bytes` bytes at `base` (raw buffer, 32-bit elements;
// out-of-range loads return 0 and out-of-range stores are dropped).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// Device-coherent record traffic for the concurrent schedule.  On this multi-die GPU
// each die's L2 is coherent only with itself; a store or load with the device-scope
// coherence bit (SC1) is written through / fetched past it.  Records written and read this
// way need no L2 write-back or invalidation between producer and consumer: the producer
// waits for its stores to complete and then raises a flag; the consumer sees the flag and
// then reads.
constexpr int kCohAux = 16;   // cache-policy bits: SC1

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
template <typename V>
__device__ __forceinline__ void rec_store16(char *rec, int off, V v, bool coherent) {
    static_assert(sizeof(V) == 16, "16-byte store");
    if (coherent)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), make_rsrc(rec, 1 << 30), off, 0,
                                               kCohAux);
    else
        *reinterpret_cast<V *>(rec + off) = v;
}
// U' and Ol^T tiles are kept as 24-bit floats: the fp32 value with its low byte rounded
// away (half up in magnitude: sign, exponent and 15 mantissa bits remain, a relative step of
// 2^-16), four values in 12 bytes, value i's three bytes at bytes 3i .. 3i + 2.  Byte
// permutes pack and unpack them (selector 0x0c gives a zero byte).
typedef unsigned u32x3 __attribute__((ext_vector_type(3)));
// (The values are bit-cast as whole vectors: a bit cast of one subscripted element of a
// vector value was compiled as a cast of element 0.)
__device__ __forceinline__ u32x3 pack24(f32x4 v) {
    const u32x4 r = __builtin_bit_cast(u32x4, v) + 0x80u;
    return u32x3{__builtin_amdgcn_perm(r[1], r[0], 0x05030201u), __builtin_amdgcn_perm(r[2], r[1], 0x06050302u),
                 __builtin_amdgcn_perm(r[3], r[2], 0x07060503u)};
}
__device__ __forceinline__ f32x4 unpack24(u32x3 d) {
    const u32x4 r = {d[0] << 8, __builtin_amdgcn_perm(d[1], d[0], 0x0504030cu), __builtin_amdgcn_perm(d[2], d[1], 0x0403020cu),
                     d[2] & 0xffffff00u};
    return __builtin_bit_cast(f32x4, r);
}
// 12 bytes of a record (coherent: device scope, as rec_store16)
__device__ __forceinline__ void rec_store12(char *rec, int off, u32x3 v, bool coherent) {
    if (coherent)
        __builtin_amdgcn_raw_buffer_store_b96(v, make_rsrc(rec, 1 << 30), off, 0, kCohAux);
    else
        __builtin_amdgcn_raw_buffer_store_b96(v, make_rsrc(rec, 1 << 30), off, 0, 0);
}
__device__ __forceinline__ u32x3 rec_load12(const char *rec, int off, bool coherent) {
    if (coherent) return __builtin_amdgcn_raw_buffer_load_b96(make_rsrc(rec, 1 << 30), off, 0, kCohAux);
    return __builtin_amdgcn_raw_buffer_load_b96(make_rsrc(rec, 1 << 30), off, 0, 0);
}

// ============================================================== chunk-local

// Index of block (c, r), c <= r, in a packed upper triangle of 4 x 4 blocks.
__host__ __device__ constexpr int tri_idx(int c, int r) { return r * (r + 1) / 2 + c; }
// Index of block (k, c), k > c, in a packed strict lower triangle of 4 x 4 blocks.
__host__ __device__ constexpr int stri_idx(int k, int c) { return k * (k - 1) / 2 + c; }

// An A or B operand that holds one 16 x 16 block (k < 16): the four values of
// this lane in the low half, zeros in the high half (see kperm).
__device__ __forceinline__ Split8 split_block(f32x4 x) { return split_tiles(x, zero4()); }
__device__ __forceinline__ Split8 block_operand(bf16x4 hi, bf16x4 lo) {
    Split8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r.hi[i] = hi[i]; r.lo[i] = lo[i];
        r.hi[4 + i] = (bf16)0.f; r.lo[4 + i] = (bf16)0.f;
    }
    return r;
}
__device__ __forceinline__ Split8 neg_split(Split8 s) { return Split8{-s.hi, -s.lo}; }
__device__ __forceinline__ void split_store(f32x4 x, bf16x4 *hi, bf16x4 *lo) {
    const float v[4] = {x[0], x[1], x[2], x[3]};
    bf16x4 h, l;
    split4(v, &h, &l);
    *hi = h;
    *lo = l;
}
__device__ __forceinline__ bf16x8 to_bf16x8(f32x4 a, f32x4 b) {   // exact when a, b hold bf16 values
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) { r[i] = (bf16)a[i]; r[4 + i] = (bf16)b[i]; }
    return r;
}

// Workgroup shape of the chunk-local kernel: D / 32 waves per half (head-dim
// tiles for W and Qt, value tiles for U and Ol), two 16-wide tiles per wave.
template <int D>
struct LocalShape {
    static constexpr int NWH = D / 32;
    static constexpr int NW = 2 * NWH;
    static constexpr int THREADS = 64 * NW;
};

// LDS layout of the chunk-local kernel (bytes).
template <int D>
struct LocalSmem {
    static constexpr int NW = LocalShape<D>::NW;
    static constexpr int LD = D + 8;                         // bf16 row stride of the K / Q planes
    static constexpr int PLANE = 64 * LD * 2;
    static constexpr int KH = 0, KL = PLANE, QH = 2 * PLANE, QL = 3 * PLANE;
    static constexpr int SCR = 0;                            // after the tile phase: per-wave solve scratch
    static constexpr int SCR_LANE = 20;                      //   floats per column (padded)
    static constexpr int SCR_WAVE = 4 * 16 * SCR_LANE * 4;
    static constexpr int ADIAG = 4 * PLANE;                  // diagonal blocks of A, row-major fp32
    static constexpr int ADIAG_BLK = 16 * 16 + 4;            //   floats per block (padded)
    static constexpr int AOFF = ADIAG + 4 * ADIAG_BLK * 4;   // strict-lower blocks of A: [6][hi, lo][64] bf16x4
    static constexpr int PT = AOFF + 6 * 2 * 64 * 8;         // P^T blocks c <= r: [10][64] f32x4
    static constexpr int XT = PT + 10 * 64 * 16;             // scaled T^T, M^T blocks c <= r: [4][10][hi, lo][64] bf16x4
    static constexpr int SCAL = XT + 4 * 10 * 2 * 64 * 8;    // token scalars: G, beta, beta e^Gr, e^{G_c - G}, e^G, Gr
    static constexpr int VLD = D + 4;                        // fused conv: fp32 v plane [64][VLD] in the XT region
    static_assert(64 * VLD * 4 <= SCAL - XT, "v plane fits in the T / M region");
    static constexpr int SIZE = SCAL + 6 * 64 * 4;
    static_assert(NW * SCR_WAVE <= 4 * PLANE, "solve scratch fits in the planes");
    // Fused prep with a 16-bit x: the next chunk's x rows (tokens -3 .. 63, the q, k and v
    // channel groups of D each) are loaded into registers while this chunk is solved and
    // written to a staging area at its end.  Staged row r is XROW contiguous bytes
    // [q | k | v]; rows 0 .. XRA - 1 sit in the plane region past the solve scratch (free
    // from the tile phase on), the rest past SIZE.  XRA * XROW is a whole number of 1 KiB
    // copies, so no copy straddles the two.
    static constexpr int XROW = 3 * D * 2;
    static constexpr int XROWS = kChunk + kConvHist;
    static constexpr int XA = NW * SCR_WAVE;
    static constexpr int XRQ = 1024 / std::gcd(XROW, 1024);
    static constexpr int XRA = (4 * PLANE - XA) / XROW / XRQ * XRQ;
    static constexpr int XB = SIZE;
    static constexpr int XCOPIES = (3 * XROWS * 2 * D + 1023) / 1024;   // 1 KiB copies
    static constexpr int SIZE_STAGED = XB + XCOPIES * 1024 - XRA * XROW;
    static_assert(XA % 16 == 0 && XB % 16 == 0 && (XRA * XROW) % 1024 == 0, "staging alignment");
    static_assert(XA + XRA * XROW <= 4 * PLANE, "staging part A fits in the planes");
    static_assert(SIZE_STAGED <= 160 * 1024, "staging fits in LDS");
};

// A lane's part in the fused prep (lane = (token group tg, 8-channel block cb): TOK tokens x
// 8 channels, the D / 8 lanes of a token group forming one row for the L2 sums).  D = 128
// (eight waves), 16-bit x: waves 0 .. 3 convolve q and k (two waves per group, 8 tokens per
// lane) and waves 4 .. 7 convolve v (4 tokens per lane), so each SIMD (waves w and w + 4)
// carries the same share.  Otherwise D / 64 waves per group take q, k and v, 8 tokens per
// lane (with fp32 rows the two lane kinds together need more registers than a wave has).
struct ConvLane {
    bool vsplit;   // this lane convolves v, 4 tokens
    bool active;   // this lane convolves at all
    int grp, cb, tl0, ch0;
};
template <int D, typename TX>
__device__ __forceinline__ ConvLane conv_lane(int wave, int lane, int h, int kh, int Hk) {
    constexpr int NW = LocalShape<D>::NW, CB = D / 8, WPG = D / 64;
    constexpr bool VSPLIT = NW == 8 && sizeof(TX) == 2;
    ConvLane c;
    c.vsplit = VSPLIT && wave >= 4;
    c.active = VSPLIT || wave < 3 * WPG;
    c.cb = lane % CB;
    const int tg = lane / CB;
    c.grp = c.vsplit ? 2 : wave / WPG;
    c.tl0 = c.vsplit ? 16 * (wave - 4) + 4 * tg : (64 / WPG) * (wave % WPG) + 8 * tg;
    c.ch0 = (c.grp == 0 ? kh * D : c.grp == 1 ? (Hk + kh) * D : 2 * Hk * D + h * D) + 8 * c.cb;
    return c;
}

// Fused prep of one lane's TOK tokens x 8 channels of group grp (0 q, 1 k, 2 v): the TOK + 3
// input rows (from the staged rows in LDS, or x, or the conv cache before the sequence
// start, else zeros), the depthwise conv + SiLU, then for q and k the L2 norm over the D / 8
// lanes of the token group, written to the bf16 hi / lo planes; v goes to the fp32 plane.
// wt holds the lane's conv weights (wt[j][i]: tap j of channel ch0 + i); with DOT2 (16-bit x
// and weights) wp holds them as bf16 pairs (wp[j][i]: taps 2j, 2j + 1) and each output is two
// two-term dot products of a weight pair with the channel's values at two consecutive tokens
// (the products of two bf16 values are exact in fp32).  Every wave calls it once: with STAGE
// its barrier separates the reads of the staging area from the plane writes that overwrite
// part of it.  Inactive lanes only take the barrier.
template <int D, typename TX, bool STAGE, int TOK, bool DOT2>
__device__ __forceinline__ void fused_conv_lane(char *smem, const TX *__restrict__ x, const TX *__restrict__ cs_in, int conv_dim, int t0, int L, int s_,
                                                bool first, bool staged, bool active, int grp, int ch0, int tl0, int cb,
                                                float l2_eps, const float (&wt)[4][8], const unsigned (&wp)[2][8]) {
    using SM = LocalSmem<D>;
    constexpr int CB = D / 8, LD = SM::LD;
    const int grp_ = TOK == 4 ? 2 : grp;   // four-token lanes convolve v only
    Raw8<TX> rows[TOK + kConvHist];
    // A full chunk with its rows staged that does not start its sequence (the common case,
    // wave-uniform): every row is a staged row, part A below XRA, part B from XRA on.
    const bool fast = STAGE && staged && !first && L == kChunk;
    if (active && fast) {
        const int cross = SM::XRA - tl0;
        const int base_a = SM::XA + tl0 * SM::XROW + grp_ * 2 * D + 16 * cb;
        const int base_b = base_a + (SM::XB - SM::XA - SM::XRA * SM::XROW);
#pragma unroll
        for (int r = 0; r < TOK + kConvHist; ++r)
            rows[r].load(reinterpret_cast<const TX *>(smem + (r >= cross ? base_b : base_a) + r * SM::XROW));
    } else if (active) {
#pragma unroll
        for (int r = 0; r < TOK + kConvHist; ++r) {
            const int tl = tl0 - kConvHist + r;
            if (tl < L && (tl >= 0 || !first)) {
                if (STAGE && staged) {
                    const int sr = tl + kConvHist;   // staged row
                    const int so = (sr < SM::XRA ? SM::XA + sr * SM::XROW : SM::XB + (sr - SM::XRA) * SM::XROW) +
                                   grp_ * 2 * D + 16 * cb;
                    rows[r].load(reinterpret_cast<const TX *>(smem + so));
                } else {
                    rows[r].load(x + (size_t)(t0 + tl) * conv_dim + ch0);
                }
            } else if (tl < 0 && cs_in) {
                rows[r].load(cs_in + ((size_t)s_ * kConvHist + (kConvHist + tl)) * conv_dim + ch0);
            } else {
                rows[r].zero();
            }
        }
    }
    if constexpr (STAGE) __syncthreads();   // staging part A is read before the planes overwrite it
    if (!active) return;
    float hw[3][8];
    if constexpr (!DOT2) {
#pragma unroll
        for (int j = 0; j < 3; ++j) rows[j].to_f32(hw[j]);
    }
#pragma unroll
    for (int i = 0; i < TOK; ++i) {
        float xt[8], y[8];
        if constexpr (!DOT2) rows[i + kConvHist].to_f32(xt);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float acc;
            if constexpr (DOT2) {
                // (x[r][e], x[r + 1][e]) as one bf16 pair: the low or high halves of the two rows'
                // words holding channels e & ~1, e | 1
                const unsigned sel = (e & 1) ? 0x07060302u : 0x05040100u;
                auto word = [&](int r) { return __builtin_bit_cast(u32x4v, rows[r].v)[e >> 1]; };
                const unsigned p01 = __builtin_amdgcn_perm(word(i + 1), word(i), sel);
                const unsigned p23 = __builtin_amdgcn_perm(word(i + 3), word(i + 2), sel);
                acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wp[0][e]),
                                                      __builtin_bit_cast(bf16x2, p01), 0.f, false);
                acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wp[1][e]),
                                                      __builtin_bit_cast(bf16x2, p23), acc, false);
            } else {
                acc = wt[0][e] * hw[0][e];
                acc = fmaf(wt[1][e], hw[1][e], acc);
                acc = fmaf(wt[2][e], hw[2][e], acc);
                acc = fmaf(wt[3][e], xt[e], acc);
            }
            y[e] = silu(acc);
            ss = fmaf(y[e], y[e], ss);
        }
        const int tl = tl0 + i;
        if (grp_ < 2) {
            ss = group_sum<CB>(ss);
            const float rn = rsqrtf(ss + l2_eps);
            float yn[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) yn[e] = y[e] * rn;
            const Split8 sp = split8(yn);
            const bf16x8 hi = sp.hi, lo = sp.lo;
            bf16 *ph = reinterpret_cast<bf16 *>(smem + (grp == 0 ? SM::QH : SM::KH));
            bf16 *pl = reinterpret_cast<bf16 *>(smem + (grp == 0 ? SM::QL : SM::KL));
            *reinterpret_cast<bf16x8 *>(ph + tl * LD + 8 * cb) = hi;
            *reinterpret_cast<bf16x8 *>(pl + tl * LD + 8 * cb) = lo;
        } else {
            float *vp = reinterpret_cast<float *>(smem + SM::XT) + tl * SM::VLD + 8 * cb;
            *reinterpret_cast<f32x4 *>(vp) = f32x4{y[0], y[1], y[2], y[3]};
            *reinterpret_cast<f32x4 *>(vp + 4) = f32x4{y[4], y[5], y[6], y[7]};
        }
        if constexpr (!DOT2) {
#pragma unroll
            for (int e = 0; e < 8; ++e) { hw[0][e] = hw[1][e]; hw[1][e] = hw[2][e]; hw[2][e] = xt[e]; }
        }
    }
}

// One workgroup per (chunk, value head), fully parallel over chunks.  With
// T = (I + A)^-1, M = P T, Dc = diag(e^{G_c - G}), Bk = diag(b e^G), Bv = diag(b):
//   -W' = -Dc T Bk K,  U' = Dc T Bv V,  Qt = diag(e^G) Q - M Bk K,  Ol = M Bv V
// (the state pass uses Delta' = Dc Delta = U' - W' S, so the per-token decay of the
// state update is already applied and the keys enter it unscaled).  Every MFMA
// output lands in the layout its consumer wants, so nothing is transposed through
// LDS element by element:
//  1. K K^T and K Q^T tiles with key block b as the A operand -> A (strict lower)
//     and P^T, scaled by the decays.  K K^T is symmetric, so A's accumulator tile
//     (k, c) is also the A-operand form of A^T block (c, k).
//  2. The four 16 x 16 diagonal blocks T_cc by forward substitution (lane (c, j)
//     owns column j of block c): with eight waves wave 0 solves them and hands them
//     to the others through LDS with a flag (no barrier); with four, every wave.
//  3. Block back substitution of (I + A^T) X = [I | P^T] gives T^T and M^T in
//     accumulator layout, one column block per chain; the blocks are published
//     with the scalings above folded in.
//  4. W waves: W'^T = K^T (Bk T^T Dc) and Qt^T = seed - K^T (Bk M^T); in
//     accumulator layout these are exactly the state pass's A-operand fragments of
//     -W' and Qt.  The K^T operand comes from the bf16 planes on MFMA (a 0/1
//     selector picks 16 head-dim columns), exactly, and is stored as is.
//     U waves: U' = (Dc T Bv) V and Ol = (M Bv) V.
// Products use two-term bf16 splits of both operands (three MFMAs each).
// FUSED: q, k, v are not inputs; the workgroup runs the depthwise conv (kernel 4) + SiLU +
// per-head L2 of q and k itself from the pre-conv input x (element type TX; conv weights TW) of its 64 tokens
// and the 3 before them ("7.6 Qwen3.5: the linear-attention hybrid", section 7.6.2; history
// from the sequence's own earlier tokens, else its conv cache, else zeros), with the same
// arithmetic as gdn_conv_qk_prep.
// Ready flags of the concurrent schedule: 64-bit values, one per (value head, chunk), set
// to the call's own value (a fixed 32-bit tag in the high word, a per-device call counter in
// the low word).  A flag counts as raised only when it holds this call's value, so the flags
// need no clearing between calls: values left by earlier calls hold older counters, and a
// fresh workspace would have to hold the exact 64-bit pattern by chance.  A call captured in
// a HIP graph replays with one value, so there the flags are cleared by a kernel first and
// every replay uses the value (kFlagTagGraph << 32) | 1, which no other call uses.
typedef unsigned long long flag_t;
constexpr unsigned kFlagTag = 0x9e3779b9u;
constexpr unsigned kFlagTagGraph = 0x7f4a7c15u;

// LDS of the chunk-local kernel
template <int D, typename TX, bool FUSED>
constexpr int local_lds_bytes() {
    return FUSED && sizeof(TX) == 2 ? LocalSmem<D>::SIZE_STAGED : LocalSmem<D>::SIZE;
}

// Arguments of the chunk-local kernel (one struct, shared with the combined kernel of the
// concurrent schedule).
template <typename TX, typename TW>
struct LocalArgs {
    const float *q, *k, *v, *g, *beta;
    const int32_t *cu;
    int N, Ttot, Hk, Hv;
    float scale;
    char *ws;
    int ncmax, g0, g1, nslots;
    const TX *x;
    const TW *conv_w;
    const TX *cs_in;
    float l2_eps;
    int order;
    flag_t *flags;
    flag_t flag_val;
    // value heads per stored K^T: the value heads of a key head share k, so with kgroup > 1
    // only a group's first head stores the K^T fragments of its records (the state pass
    // reads them from there)
    int kgroup;
};

// The chunk-local work of workgroup (slot, value head h): smem is the workgroup's LDS
// (local_lds_bytes), tflag_ one LDS word.
template <int D, bool FUSED, typename TX, typename TW>
__device__ __forceinline__ void chunk_local_body(char *smem, int *tflag_, int slot, int h, const LocalArgs<TX, TW> &P) {
    using R = Rec<D>;
    using SM = LocalSmem<D>;
    constexpr bool STAGE = FUSED && sizeof(TX) == 2;
    constexpr int NWH = LocalShape<D>::NWH, NW = LocalShape<D>::NW, NT = LocalShape<D>::THREADS;
    constexpr int NKS = D / 32;   // 32-wide k steps over the head dim
    constexpr int LD = SM::LD;
    constexpr int NF_K = (D / 16) * 2;
    const float *__restrict__ q = P.q, *__restrict__ k = P.k, *__restrict__ v = P.v;
    const float *__restrict__ g = P.g, *__restrict__ beta = P.beta;
    const int32_t *__restrict__ cu = P.cu;
    const int N = P.N, Ttot = P.Ttot, Hk = P.Hk, Hv = P.Hv, ncmax = P.ncmax, g0 = P.g0, g1 = P.g1;
    const int nslots = P.nslots, order = P.order;
    const float scale = P.scale, l2_eps = P.l2_eps;
    char *__restrict__ ws = P.ws;
    const TX *__restrict__ x = P.x;
    const TW *__restrict__ conv_w = P.conv_w;
    const TX *__restrict__ cs_in = P.cs_in;
    flag_t *flags = P.flags;
    const flag_t flag_val = P.flag_val;
    int &tflag = *tflag_;   // diagonal blocks of the current chunk published (value: chunk + 1)
    if (threadIdx.x == 0) tflag = -1;   // seen by every wave after the chunk loop's first barrier
    bf16 *Kh = reinterpret_cast<bf16 *>(smem + SM::KH);
    bf16 *Kl = reinterpret_cast<bf16 *>(smem + SM::KL);
    bf16 *Qh = reinterpret_cast<bf16 *>(smem + SM::QH);
    bf16 *Ql = reinterpret_cast<bf16 *>(smem + SM::QL);
    float *Adiag = reinterpret_cast<float *>(smem + SM::ADIAG);
    bf16x4 *Aoff = reinterpret_cast<bf16x4 *>(smem + SM::AOFF);     // [6][2][64]
    f32x4 *Pt = reinterpret_cast<f32x4 *>(smem + SM::PT);           // [10][64]
    bf16x4 *Xt = reinterpret_cast<bf16x4 *>(smem + SM::XT);         // [4][10][2][64]
    float *Gs = reinterpret_cast<float *>(smem + SM::SCAL);
    float *Bs = Gs + 64, *BEG = Gs + 128, *DCs = Gs + 192, *QS = Gs + 256, *GRs = Gs + 320;
    enum { XT_TW = 0, XT_TU = 1, XT_MW = 2, XT_MU = 3 };   // published operand sets

    const int kh = h / (Hv / Hk);
    const int conv_dim = 2 * Hk * D + Hv * D;

    // Persistent over chunks: workgroup (slot, head) takes packed chunks g0 + slot,
    // g0 + slot + nslots, ... of its head, so one workgroup per compute unit runs the
    // whole launch and (fused, 16-bit x) loads the next chunk's x while solving this one.
    bool staged = false;   // this chunk's x rows are in the LDS staging area
    // Where the chunk lives: sequence s_, its chunk c_, the sequence's token range [sb, se).
    // Carried from one iteration to the next; searched for only when the next chunk lies
    // in another sequence.
    int s_ = 0, c_ = 0, sb = 0, se = 0;
    bool have = false;
    // Fused: the lane's conv weights, loaded once (a workgroup keeps its head, so its lanes
    // keep their channels, for the whole launch).
    // With 16-bit x and weights the taps go in pairs: cwp[j][i] holds taps 2j, 2j + 1 of
    // channel ch0 + i as a bf16 pair (low half first), for two-term dot products.
    constexpr bool DOT2 = STAGE && sizeof(TW) == 2;
    float cwt[4][8];
    unsigned cwp[2][8];
    if constexpr (FUSED) {
        const ConvLane cl = conv_lane<D, TX>(threadIdx.x >> 6, threadIdx.x & 63, h, kh, Hk);
        if constexpr (DOT2) {
            // A channel's four bf16 taps are 8 contiguous bytes: its words (taps 0, 1) and
            // (taps 2, 3) are already the pairs, low half first.  Four 16-byte loads cover the
            // lane's 8 channels; nothing waits for them before the first conv.
            const u32x4 *cw4 = reinterpret_cast<const u32x4 *>(conv_w + (size_t)cl.ch0 * kConvK);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const u32x4 w = cl.active ? cw4[q4] : u32x4{0u, 0u, 0u, 0u};
                cwp[0][2 * q4] = w[0]; cwp[1][2 * q4] = w[1];
                cwp[0][2 * q4 + 1] = w[2]; cwp[1][2 * q4 + 1] = w[3];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) cwt[j][i] = 0.f;   // not used with the pairs
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    cwt[j][i] = cl.active ? to_f32(conv_w[(size_t)(cl.ch0 + i) * kConvK + j]) : 0.f;
        }
    }
    for (int gc = g0 + slot; gc < g1; gc += nslots) {
    // The thread index passes through an empty asm each iteration, so nothing derived from
    // it is hoisted out of the loop and kept live across it (that costs registers the
    // chunk's own work needs).
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    // wave index in a scalar register: wave-level branches and LDS bases stay uniform
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, kg = lane >> 4;
    const bool isW = wave < NWH;
    const int qw = isW ? wave : wave - NWH;   // this wave's pair of 16-wide tiles: 2qw, 2qw + 1
    // ---- where this chunk lives (every wave finds the same answer; no barrier)
    if (!have && !locate_chunk_wave(cu, N, Ttot, gc, s_, c_, sb, se)) break;
    const int t0 = sb + c_ * kChunk;
    const int L = min(kChunk, se - t0);
    char *rec = ws + ((size_t)h * ncmax + gc) * R::SIZE;   // head-major: a head's chunks are contiguous

    // ---- global loads, all issued before any is used.  Rows >= L are clamped
    // (loads stay in bounds and unconditional) and zeroed.
    constexpr int NV = FUSED ? 1 : 64 * (D / 4) / NT;
    float4 kv[NV], qv[NV];
#pragma unroll
    for (int i = 0; i < NV && !FUSED; ++i) {
        const int e = tid + NT * i, r = e / (D / 4), c4 = (e % (D / 4)) * 4;
        const size_t off = ((size_t)(t0 + min(r, L - 1)) * Hk + kh) * D + c4;
        kv[i] = *reinterpret_cast<const float4 *>(k + off);
        qv[i] = *reinterpret_cast<const float4 *>(q + off);
    }
    // W waves: Q^T in accumulator layout (rows = head dim, cols = token) seeds Qt^T.
    // U waves: V in accumulator layout (rows = token) feeds U' and Ol.
    f32x4 Xa[2][4];
    if (FUSED) {
        // filled from the planes after the conv (below)
    } else if (isW) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const int t = 16 * tt + l16, d = 16 * (2 * qw + mi) + 4 * kg;
                const float4 x = *reinterpret_cast<const float4 *>(q + ((size_t)(t0 + min(t, L - 1)) * Hk + kh) * D + d);
                Xa[mi][tt] = t < L ? f32x4{x.x, x.y, x.z, x.w} : zero4();
            }
    } else {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * rt + 4 * kg + r, col = 16 * (2 * qw + ni) + l16;
                    const float x = v[((size_t)(t0 + min(t, L - 1)) * Hv + h) * D + col];
                    Xa[ni][rt][r] = t < L ? x : 0.f;
                }
    }
    if (wave == (FUSED ? NW - 1 : 0)) {
        const int rr = min(lane, L - 1);
        const float g0 = g[(size_t)(t0 + rr) * Hv + h], b0 = beta[(size_t)(t0 + rr) * Hv + h];
        const float gg = lane < L ? g0 : 0.f, bb = lane < L ? b0 : 0.f;
        float G = gg;   // inclusive prefix sum over the chunk
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_up(G, o, kWave);
            if (lane >= o) G += y;
        }
        const float Gc = __shfl(G, 63, kWave);
        const float eg = __expf(G);
        // decay seen by the retrieval of token t: G_t, or G_{t-1} = G_t - g_t when the
        // retrieval reads the state before the decay (order 1)
        const float Gr = order == 0 ? G : G - gg;
        Gs[lane] = G;
        GRs[lane] = Gr;
        Bs[lane] = bb;
        BEG[lane] = bb * (order == 0 ? eg : __expf(Gr));
        DCs[lane] = __expf(Gc - G);
        QS[lane] = eg;
        if (lane < 5) {   // e^{G_c} four times, then the query scale (applied by the state pass)
            const float val = lane < 4 ? __expf(Gc) : scale;
            if (flags)
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, val), make_rsrc(rec, 1 << 30),
                                                      R::GM_OFF + 4 * lane, 0, kCohAux);
            else
                reinterpret_cast<float *>(rec + R::GM_OFF)[lane] = val;
        }
    }
    if constexpr (FUSED) {
        // conv + SiLU + L2 from x (lane roles: conv_lane).  Tokens past the chunk's last one
        // (a sequence's last chunk) get finite values that no stored result depends on: their
        // beta and g are 0, so their rows of A, W' and U' are exactly zero (T's row is the
        // identity row), Delta' vanishes there and their outputs are not stored.
        const ConvLane cl = conv_lane<D, TX>(wave, lane, h, kh, Hk);
        const bool first = c_ == 0;              // history before the sequence start
        if (cl.vsplit)
            fused_conv_lane<D, TX, STAGE, 4, DOT2>(smem, x, cs_in, conv_dim, t0, L, s_, first, staged, true, cl.grp,
                                                   cl.ch0, cl.tl0, cl.cb, l2_eps, cwt, cwp);
        else
            fused_conv_lane<D, TX, STAGE, 8, DOT2>(smem, x, cs_in, conv_dim, t0, L, s_, first, staged, cl.active,
                                                   cl.grp, cl.ch0, cl.tl0, cl.cb, l2_eps, cwt, cwp);
    }
    // K and Q as bf16 hi / lo planes, row-major [token][head dim]
#pragma unroll
    for (int i = 0; i < NV && !FUSED; ++i) {
        const int e = tid + NT * i, r = e / (D / 4), c4 = (e % (D / 4)) * 4;
        const bool live = r < L;
        const float kk[4] = {kv[i].x, kv[i].y, kv[i].z, kv[i].w};
        const float qq[4] = {qv[i].x, qv[i].y, qv[i].z, qv[i].w};
        float ka4[4], qa4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ka4[j] = live ? kk[j] : 0.f;
            qa4[j] = live ? qq[j] : 0.f;
        }
        bf16x4 khi, klo, qhi, qlo;
        split4(ka4, &khi, &klo);
        split4(qa4, &qhi, &qlo);
        *reinterpret_cast<bf16x4 *>(Kh + r * LD + c4) = khi;
        *reinterpret_cast<bf16x4 *>(Kl + r * LD + c4) = klo;
        *reinterpret_cast<bf16x4 *>(Qh + r * LD + c4) = qhi;
        *reinterpret_cast<bf16x4 *>(Ql + r * LD + c4) = qlo;
    }
    __syncthreads();

    // ---- 1. tiles with key block b as the A operand: K K^T (b, c <= b) and K Q^T (b, r >= b),
    // five in all, numbered j = 0 .. 4 (K K^T c = j for j <= b, then K Q^T r = j - 1).
    // Eight waves: wave b takes tiles 0 and 1 of block b and wave 4 + b tiles 2 .. 4 (the W
    // waves have the heavier work after this phase); four waves: wave b takes all five.
    // The tile loops run at compile time (one instance per key block), so the next tile's
    // operand reads are issued under the current tile's MFMAs.
    {
        const int b = wave & 3;
        auto tiles = [&](auto btag, auto lotag, auto hitag) __attribute__((always_inline)) {
            constexpr int B = decltype(btag)::value;
            constexpr int j0 = decltype(lotag)::value, j1 = decltype(hitag)::value;   // tiles [j0, j1)
            Split8 ka[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int off = (16 * B + l16) * LD + 32 * ks + 8 * kg;
                ka[ks] = Split8{*reinterpret_cast<const bf16x8 *>(Kh + off),
                                *reinterpret_cast<const bf16x8 *>(Kl + off)};
            }
            if constexpr (j0 <= B) {
                const f32x4 Bb = *reinterpret_cast<const f32x4 *>(Bs + 16 * B + 4 * kg);
                const f32x4 Grb = *reinterpret_cast<const f32x4 *>(GRs + 16 * B + 4 * kg);
#pragma unroll
                for (int c = 0; c <= B; ++c) {
                    if (c < j0 || c >= j1) continue;
                    Acc3 s3 = acc3_zero();
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        const int off = (16 * c + l16) * LD + 32 * ks + 8 * kg;
                        const Split8 kb{*reinterpret_cast<const bf16x8 *>(Kh + off),
                                        *reinterpret_cast<const bf16x8 *>(Kl + off)};
                        mfma3_acc(s3, ka[ks], kb);
                    }
                    const f32x4 acc = acc3_sum(s3);
                    // A[t][i] = b_t e^{Gr_t - G_i} k_t . k_i for i < t; t = 16B + 4kg + r, i = 16c + l16
                    const int i = 16 * c + l16;
                    const float Gi = Gs[i];
                    f32x4 a;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = 16 * B + 4 * kg + r;
                        a[r] = i < t ? Bb[r] * __expf(Grb[r] - Gi) * acc[r] : 0.f;
                    }
                    if (c == B) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) Adiag[c * SM::ADIAG_BLK + (4 * kg + r) * 16 + l16] = a[r];
                    } else {
                        const int s = stri_idx(B, c);
                        split_store(a, &Aoff[(s * 2 + 0) * 64 + lane], &Aoff[(s * 2 + 1) * 64 + lane]);
                    }
                }
            }
            if constexpr (j1 > B + 1) {
                const f32x4 Gb = *reinterpret_cast<const f32x4 *>(Gs + 16 * B + 4 * kg);
#pragma unroll
                for (int r = B; r < 4; ++r) {
                    if (r + 1 < j0 || r + 1 >= j1) continue;
                    Acc3 s3 = acc3_zero();
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        const int off = (16 * r + l16) * LD + 32 * ks + 8 * kg;
                        const Split8 qb{*reinterpret_cast<const bf16x8 *>(Qh + off),
                                        *reinterpret_cast<const bf16x8 *>(Ql + off)};
                        mfma3_acc(s3, ka[ks], qb);
                    }
                    const f32x4 acc = acc3_sum(s3);
                    // P^T[i][t] = e^{G_t - G_i} q_t . k_i for i <= t; i = 16B + 4kg + rr, t = 16r + l16
                    const int t = 16 * r + l16;
                    const float Gt = Gs[t];
                    f32x4 p;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int i = 16 * B + 4 * kg + rr;
                        p[rr] = i <= t ? __expf(Gt - Gb[rr]) * acc[rr] : 0.f;
                    }
                    Pt[tri_idx(B, r) * 64 + lane] = p;
                }
            }
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        using I3 = std::integral_constant<int, 3>;
        using I5 = std::integral_constant<int, 5>;
        if constexpr (NW == 4) {
            switch (b) {
            case 0: tiles(I0{}, I0{}, I5{}); break;
            case 1: tiles(I1{}, I0{}, I5{}); break;
            case 2: tiles(I2{}, I0{}, I5{}); break;
            default: tiles(I3{}, I0{}, I5{}); break;
            }
        } else {
            switch (wave) {
            case 0: tiles(I0{}, I0{}, I2{}); break;
            case 1: tiles(I1{}, I0{}, I2{}); break;
            case 2: tiles(I2{}, I0{}, I2{}); break;
            case 3: tiles(I3{}, I0{}, I2{}); break;
            case 4: tiles(I0{}, I2{}, I5{}); break;
            case 5: tiles(I1{}, I2{}, I5{}); break;
            case 6: tiles(I2{}, I2{}, I5{}); break;
            default: tiles(I3{}, I2{}, I5{}); break;
            }
        }
    }
    // W waves: K in accumulator layout (rows = token) for head-dim tiles 2qw, 2qw + 1, on
    // MFMA from the row fragments: D = K_rows x Sel with Sel[k][j] = (k == 16 hh + j).  The hi
    // and lo planes go through separately, so the results are exact bf16 values and form the
    // K^T operand (lane row = head dim, k = token in kperm order) with no rounding.  They go to
    // the record as they are and stay as this wave's A operand of step 4.
    // U waves: V as B operands (k = token in kperm order).
    if constexpr (FUSED) {
        if (isW) {   // Q^T seed from the q planes (hi + lo)
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const int off = (16 * tt + l16) * LD + 16 * (2 * qw + mi) + 4 * kg;
                    const bf16x4 a = *reinterpret_cast<const bf16x4 *>(Qh + off);
                    const bf16x4 b = *reinterpret_cast<const bf16x4 *>(Ql + off);
#pragma unroll
                    for (int e = 0; e < 4; ++e) Xa[mi][tt][e] = (float)a[e] + (float)b[e];
                }
        } else {     // V in accumulator layout from the fp32 v plane
            const float *vp = reinterpret_cast<const float *>(smem + SM::XT);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        Xa[ni][rt][r] = vp[(16 * rt + 4 * kg + r) * SM::VLD + 16 * (2 * qw + ni) + l16];
        }
    }
    Split8 Bop[2][2];   // [tile][token k step]
    if (isW) {
        bf16x8 sel[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int vv = 0; vv < 8; ++vv) sel[hh][vv] = (bf16)((8 * kg + vv == 16 * hh + l16) ? 1.f : 0.f);
        f32x4 Kth[4][2], Ktl[4][2];   // [token block][tile]
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const int off = (16 * rt + l16) * LD + 32 * qw + 8 * kg;
            const bf16x8 kh8 = *reinterpret_cast<const bf16x8 *>(Kh + off);
            const bf16x8 kl8 = *reinterpret_cast<const bf16x8 *>(Kl + off);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                Kth[rt][hh] = mfma16(kh8, sel[hh], zero4());
                Ktl[rt][hh] = mfma16(kl8, sel[hh], zero4());
            }
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int m = 2 * qw + hh;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                Bop[hh][kt] = Split8{to_bf16x8(Kth[2 * kt][hh], Kth[2 * kt + 1][hh]),
                                     to_bf16x8(Ktl[2 * kt][hh], Ktl[2 * kt + 1][hh])};
                const int off = R::K_OFF + ((m * 2 + kt) * 64 + lane) * 16;
                if (h % P.kgroup == 0) {
                    rec_store16(rec, off, Bop[hh][kt].hi, flags != nullptr);
                    rec_store16(rec, off + NF_K * 64 * 16, Bop[hh][kt].lo, flags != nullptr);
                }
            }
        }
    } else {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) Bop[ni][kt] = split_tiles(Xa[ni][2 * kt], Xa[ni][2 * kt + 1]);
    }
    __syncthreads();

    // ---- fused prep, 16-bit x: stage the next chunk's x rows (its tokens -3 .. 63) in LDS,
    // spread over all waves.  Copy i (1 KiB) fills staging bytes [1 KiB i, 1 KiB (i + 1));
    // lane l moves 16 bytes of segment (row, group) = (i * SPI + l / SEGL) / 3.  Rows before
    // the buffer start or past its end read as 0 (they are not used: history rows of a
    // sequence's first chunk come from its conv cache, rows past its last token feed only
    // tokens on which no stored result depends).
    // The next chunk of this workgroup: chunk c_ + nslots of the same sequence if it has
    // one, else found by a search.
    const int gn = gc + nslots;
    int sn = s_, cn = c_ + nslots, sbn = sb, sen = se;
    bool next_ok = false;
    if (gn < g1) {
        if (cn * kChunk < se - sb) {
            next_ok = true;
        } else if (locate_chunk_wave(cu, N, Ttot, gn, sn, cn, sbn, sen)) {
            next_ok = true;
        }
    }
    // Eight waves: wave 0 alone solves the diagonal blocks (one wave's 64 lanes cover all
    // four) and hands them over through LDS with a flag, while the other waves go on.
    constexpr bool ONE_SOLVER = NW == 8;
    float *scr = reinterpret_cast<float *>(smem + SM::SCR + (ONE_SOLVER ? 0 : wave) * SM::SCR_WAVE);
    if (!ONE_SOLVER || wave == 0) {
        const int c = kg, j = l16;
        const float *Ab = Adiag + c * SM::ADIAG_BLK;
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float s0 = (t == j) ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
            for (int i4 = 0; i4 < t; i4 += 4) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(Ab + t * 16 + i4);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (i4 + e < t) {
                        if (e & 1) s1 = fmaf(-a[e], x[i4 + e], s1);
                        else s0 = fmaf(-a[e], x[i4 + e], s0);
                    }
            }
            x[t] = s0 + s1;
        }
#pragma unroll
        for (int t4 = 0; t4 < 16; t4 += 4)
            *reinterpret_cast<f32x4 *>(scr + (c * 16 + j) * SM::SCR_LANE + t4) =
                f32x4{x[t4], x[t4 + 1], x[t4 + 2], x[t4 + 3]};
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the scratch writes are done
        if (ONE_SOLVER) __hip_atomic_store(&tflag, gc + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    // Staging by registers, not direct-to-LDS loads: after a direct-to-LDS load the compiler
    // makes the wave's next LDS access wait for it, which would put the load's whole memory
    // latency in the middle of this chunk.  Plain loads are waited for only where their
    // registers are read, at the end of this chunk when they are written to LDS.
    constexpr int XPW = (SM::XCOPIES + NW - 1) / NW;   // 16-byte loads per lane
    u32x4 xst[STAGE ? XPW : 1];
    if constexpr (STAGE) {
        if (next_ok) {
            constexpr int SEGL = 2 * D / 16, SPI = 64 / SEGL;
            // wave-uniform (scalar) so that the buffer resource is one scalar descriptor
            const int tn = __builtin_amdgcn_readfirstlane(sbn + cn * kChunk);
            const int rb = max(tn - kConvHist, 0);
            const long bytes = (long)(Ttot - rb) * conv_dim * 2;
            const __amdgpu_buffer_rsrc_t rx =
                make_rsrc(x + (size_t)rb * conv_dim, (int)min(bytes, (long)0x7ffffff0));
#pragma unroll
            for (int k = 0; k < XPW; ++k) {
                const int i = wave + k * NW;
                if (i < SM::XCOPIES) {
                    const int sg = i * SPI + lane / SEGL;
                    const int r = min(sg / 3, SM::XROWS - 1), gi = sg % 3;
                    const int chb = gi == 0 ? kh * D : gi == 1 ? (Hk + kh) * D : 2 * Hk * D + h * D;
                    const int voff = ((tn - kConvHist + r - rb) * conv_dim + chb) * 2 + 16 * (lane % SEGL);
                    xst[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, voff, 0, 0);
                }
            }
        }
    }

    if (ONE_SOLVER && wave != 0) {
        // wave 0 raises the flag unconditionally a few thousand cycles after the barrier; the
        // bound only keeps a broken invariant from hanging the kernel
        for (int it = 0; it < (1 << 20); ++it) {
            if (__hip_atomic_load(&tflag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == gc + 1) break;
            __builtin_amdgcn_s_sleep(1);
        }
        asm volatile("" ::: "memory");
    }
    Split8 Tcc[4];   // A-operand form of T_cc^T (= accumulator layout of T_cc)
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
        Tcc[cc] = split_block(*reinterpret_cast<const f32x4 *>(scr + (cc * 16 + l16) * SM::SCR_LANE + 4 * kg));
    // ---- 3. back substitution (I + A^T) X = [I | P^T], one column block per chain:
    //   X_cr = T_cc^T (RHS_cr - sum_{k = c+1..r} (A^T)_ck X_kr),  c = r, r-1, .., 0
    // chains 0..3: column blocks of T^T (RHS = I); chains 4..7: column blocks of M^T.
    auto aT = [&](int kk, int c) __attribute__((always_inline)) {   // A-operand form of (A^T)_{c,kk}: accumulator tile (kk, c) of A
        const int s = stri_idx(kk, c);
        return block_operand(Aoff[(s * 2 + 0) * 64 + lane], Aoff[(s * 2 + 1) * 64 + lane]);
    };
    // Publish block (c, r) (rows t' = 16c + 4kg + i, column t = 16r + l16) of a scaled copy.
    auto publish = [&](int set, int c, int r, f32x4 x, const float *rowscale, float colscale) __attribute__((always_inline)) {
        const f32x4 rs = *reinterpret_cast<const f32x4 *>(rowscale + 16 * c + 4 * kg);
        const int s = (set * 10 + tri_idx(c, r)) * 2;
        split_store(x * rs * colscale, &Xt[(s + 0) * 64 + lane], &Xt[(s + 1) * 64 + lane]);
    };
    // Right-looking: as soon as block X_kr is known it is split once and its products with
    // (A^T)_ck go into every pending accumulator, the one of block k - 1 first (it gates
    // the next step of the chain), and the block is published while those MFMAs run.
    auto solve_T = [&](auto rtag) __attribute__((always_inline)) {
        constexpr int r = decltype(rtag)::value;
        bf16x8 eye;
#pragma unroll
        for (int vv = 0; vv < 8; ++vv) eye[vv] = (bf16)((vv < 4 && 4 * kg + vv == l16) ? 1.f : 0.f);
        f32x4 X = mfma16(Tcc[r].lo, eye, mfma16(Tcc[r].hi, eye, zero4()));   // T_rr^T
        f32x4 acc[4];
#pragma unroll
        for (int c = 0; c < r; ++c) acc[c] = zero4();
        const float dc = DCs[16 * r + l16];
#pragma unroll
        for (int k = r; k >= 0; --k) {
            if (k > 0) {
                const Split8 xs = split_block(X);
#pragma unroll
                for (int c = k - 1; c >= 0; --c) acc[c] = mfma16x3(aT(k, c), xs, acc[c]);
            }
            publish(XT_TW, k, r, X, BEG, dc);
            publish(XT_TU, k, r, X, Bs, dc);
            if (k > 0) X = mfma16x3p(Tcc[k - 1], split_block(-acc[k - 1]));
        }
    };
    auto solve_M = [&](auto rtag) __attribute__((always_inline)) {
        constexpr int r = decltype(rtag)::value;
        f32x4 acc[4];
#pragma unroll
        for (int c = 0; c <= r; ++c) acc[c] = Pt[tri_idx(c, r) * 64 + lane];
        f32x4 X = mfma16x3p(Tcc[r], split_block(acc[r]));
#pragma unroll
        for (int k = r; k >= 0; --k) {
            if (k > 0) {
                const Split8 xs = split_block(-X);
#pragma unroll
                for (int c = k - 1; c >= 0; --c) acc[c] = mfma16x3(aT(k, c), xs, acc[c]);
            }
            publish(XT_MW, k, r, X, BEG, 1.f);
            publish(XT_MU, k, r, X, Bs, 1.f);
            if (k > 0) X = mfma16x3p(Tcc[k - 1], split_block(acc[k - 1]));
        }
    };
    auto run_chain = [&](int ch) __attribute__((always_inline)) {
        switch (ch) {
        case 0: solve_T(std::integral_constant<int, 0>{}); break;
        case 1: solve_T(std::integral_constant<int, 1>{}); break;
        case 2: solve_T(std::integral_constant<int, 2>{}); break;
        case 3: solve_T(std::integral_constant<int, 3>{}); break;
        case 4: solve_M(std::integral_constant<int, 0>{}); break;
        case 5: solve_M(std::integral_constant<int, 1>{}); break;
        case 6: solve_M(std::integral_constant<int, 2>{}); break;
        default: solve_M(std::integral_constant<int, 3>{}); break;
        }
    };
    if (NW == 8) {
        // waves w and w + 4 share a SIMD: T chain w with M chain 3 - w keeps the long chains apart
        run_chain(wave < 4 ? wave : 11 - wave);
    } else {   // four waves: long and short chains paired
        run_chain(3 - wave);
        run_chain(4 + wave);
    }
    __syncthreads();

    // ---- 4. the four products.  Row fragment (tt, ks) of a published set: lane row
    // t = 16 tt + l16, k = t' = 32 ks + kperm(kg, v), i.e. blocks (2ks, tt), (2ks + 1, tt).
    auto row_frag = [&](int set, int tt, int ks) __attribute__((always_inline)) {
        Split8 f;
        const int b0 = (set * 10 + tri_idx(2 * ks, tt)) * 2;
        const bf16x4 h0 = Xt[b0 * 64 + lane], l0 = Xt[(b0 + 1) * 64 + lane];
        bf16x4 h1, l1;
        if (2 * ks + 1 <= tt) {
            const int b1 = (set * 10 + tri_idx(2 * ks + 1, tt)) * 2;
            h1 = Xt[b1 * 64 + lane];
            l1 = Xt[(b1 + 1) * 64 + lane];
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) { h1[i] = (bf16)0.f; l1[i] = (bf16)0.f; }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f.hi[i] = h0[i]; f.hi[4 + i] = h1[i];
            f.lo[i] = l0[i]; f.lo[4 + i] = l1[i];
        }
        return f;
    };
    // Each wave forms its first product tile by tile and stores every tile as soon as it is
    // complete, so the stores drain while the second product runs.  The three partial products
    // of each split product accumulate separately (six independent MFMA chains per step).
    if (isW) {
        // W'^T = K^T (Bk T^T Dc), stored negated as fp16 A fragments
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            Acc3 y[2] = {acc3_zero(), acc3_zero()};
#pragma unroll
            for (int ks = 0; 2 * ks <= tt; ++ks) {
                const Split8 ft = row_frag(XT_TW, tt, ks);
#pragma unroll
                for (int mi = 0; mi < 2; ++mi) mfma3_acc(y[mi], Bop[mi][ks], ft);
            }
            const int off = ((tt * NKS + qw) * 64 + lane) * 16;
            rec_store16(rec, R::W_OFF + off, pack_h(-acc3_sum(y[0]), -acc3_sum(y[1])), flags != nullptr);
        }
        // Qt^T = e^G Q^T - K^T (Bk M^T)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const float qs = QS[16 * tt + l16];
            Acc3 x[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) x[mi] = Acc3{Xa[mi][tt] * qs, zero4(), zero4()};
#pragma unroll
            for (int ks = 0; 2 * ks <= tt; ++ks) {
                const Split8 fm = neg_split(row_frag(XT_MW, tt, ks));
#pragma unroll
                for (int mi = 0; mi < 2; ++mi) mfma3_acc(x[mi], Bop[mi][ks], fm);
            }
            const int off = ((tt * NKS + qw) * 64 + lane) * 16;
            rec_store16(rec, R::Q_OFF + off, pack_h(acc3_sum(x[0]), acc3_sum(x[1])), flags != nullptr);
        }
    } else {
        // U' = (Dc T Bv) V, then Ol^T = V^T (M Bv)^T (formed transposed: the A form of V^T and
        // the B form of (M Bv)^T are the fragments at hand, and the state pass, which forms O^T
        // the same way, then holds 4 consecutive columns of one output row per lane)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            Acc3 y[2] = {acc3_zero(), acc3_zero()};
#pragma unroll
            for (int ks = 0; 2 * ks <= rt; ++ks) {
                const Split8 ft = row_frag(XT_TU, rt, ks);
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) mfma3_acc(y[ni], ft, Bop[ni][ks]);
            }
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                rec_store12(rec, R::U_OFF + (((2 * qw + ni) * 4 + rt) * 64 + lane) * 12, pack24(acc3_sum(y[ni])),
                            flags != nullptr);
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            Acc3 x[2] = {acc3_zero(), acc3_zero()};
#pragma unroll
            for (int ks = 0; 2 * ks <= rt; ++ks) {
                const Split8 fm = row_frag(XT_MU, rt, ks);
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) mfma3_acc(x[ni], Bop[ni][ks], fm);
            }
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                rec_store12(rec, R::O_OFF + (((2 * qw + ni) * 4 + rt) * 64 + lane) * 12, pack24(acc3_sum(x[ni])),
                            flags != nullptr);
        }
    }
    // the next chunk's x rows into the staging area (copy i fills staging bytes [1 KiB i,
    // 1 KiB (i + 1)), lane l the 16 bytes at 16 l)
    if constexpr (STAGE) {
        if (next_ok) {
#pragma unroll
            for (int k = 0; k < XPW; ++k) {
                const int i = wave + k * NW;
                if (i < SM::XCOPIES) {
                    char *dst = i * 1024 < SM::XRA * SM::XROW ? smem + SM::XA + i * 1024
                                                              : smem + SM::XB + (i * 1024 - SM::XRA * SM::XROW);
                    *reinterpret_cast<u32x4 *>(dst + 16 * lane) = xst[k];
                }
            }
        }
    }
    // Publishing (a state pass runs concurrently and waits for each record): the record
    // stores are device-coherent; every wave waits until its own have completed, then one
    // thread raises the chunk's flag.
    if (flags) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();   // the next chunk rewrites the planes, the T / M operands and the scalars
    if (flags && tid == 0)
        __hip_atomic_store(flags + (size_t)h * ncmax + gc, flag_val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!next_ok) break;
    s_ = sn;
    c_ = cn;
    sb = sbn;
    se = sen;
    have = true;
    staged = STAGE && next_ok;
    }
}

template <int D, bool FUSED, typename TX, typename TW = TX>
__global__ __launch_bounds__(LocalShape<D>::THREADS) void chunk_local_kernel(LocalArgs<TX, TW> P) {
    __shared__ __attribute__((aligned(16))) char smem[local_lds_bytes<D, TX, FUSED>()];
    __shared__ int tflag;
    chunk_local_body<D, FUSED, TX, TW>(smem, &tflag, blockIdx.x, blockIdx.y, P);
}

// ============================================================== state pass

// Copy `bytes` (a multiple of 1 KiB) at byte `src_off` of the buffer to LDS:
// each wave instruction moves 1 KiB (lane l -> base + 16 l); completion is
// tracked by vmcnt.  Addresses are all scalar except the constant lane offset.
// The block order is rotated by `rot` so that workgroups copying the same
// record at the same time touch different L2 lines.
template <int AUX>
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t r, int src_off, char *dst, int bytes, int lane,
                                            int rot = 0) {
    const int nblk = bytes / 1024;
#pragma unroll 8
    for (int i = 0; i < nblk; ++i) {
        int blk = i + rot;
        blk = blk >= nblk ? blk - nblk : blk;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(dst + blk * 1024), 16,
                                                 lane * 16, src_off + blk * 1024, 0, AUX);
    }
}

// One 4-wave workgroup per (sequence, value head, pair of 16-column strips of
// the state).  Waves 0 and 1 compute one strip each; waves 2 and 3 only copy.
// A strip's fp32 state lives in MFMA accumulators for the whole sequence.  Each
// chunk's A operands (W, Qt, K^T hi / lo fragments: the first Rec::U_OFF bytes
// of its record, shared by all strips of the head and kept in L2 by placing
// those workgroups on one XCD) are staged in LDS by the copy waves,
// double-buffered, while the compute waves work on the previous chunk: a single
// wave keeps too few requests in flight to stream a record at memory latency,
// and a wave with direct-to-LDS loads in flight cannot wait on its own LDS reads
// precisely.  The compute waves prefetch their strip's U and Ol tiles one chunk
// ahead into registers and read fragments from LDS in groups of 16; the next group's
// reads are issued right after the first MFMAs of the current one, and every group
// runs four independent MFMA chains (a dependent MFMA waits ~44 cycles, one issues
// every 16).  Delta' of all four row tiles comes first, then the outputs, so that the
// split of Delta' into bf16 hi / lo runs among the output MFMAs.
// Bound on the state pass's wait for a published record (iterations of a ~128-cycle
// sleep, about a second).  A wait that runs out marks the call failed: the status word
// of the workspace reports GDN_ERR_TIMEOUT and the outputs of the chunks not yet done and
// the final state are written as NaN, so a producer that never publishes ends in a
// reported failure, never in a hang or in plausible-looking output.
constexpr int kSpinMax = 1 << 24;

// The workspace status word (first 8 bytes of the workspace header): a kernel that meets
// a failure stores (kStatusTag << 32) | gdn status code; only the host clears it.
__device__ __forceinline__ void report_status(unsigned long long *status, unsigned code) {
    __hip_atomic_store(status, ((unsigned long long)kStatusTag << 32) | code, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Conv-cache write of the fused prefill, done by the state pass in the concurrent schedule:
// the three rows before the end of sequence s (x rows, or input-cache rows where the
// sequence is shorter than three tokens, or zeros without an input cache), for the
// channels [ch0, ch0 + n).  One lane per channel reads its three values before writing
// any, so the output cache may alias the input cache.  E is the element's bit pattern.
struct ConvOut {
    const void *x = nullptr;
    const void *cs_in = nullptr;
    void *cs_out = nullptr;   // nullptr: no conv cache to write
    int esz = 0;              // element bytes (2 or 4)
    int conv_dim = 0, Hk = 0, G = 1, dk = 0;
};

template <typename E>
__device__ __forceinline__ void conv_rows_copy(const ConvOut &cv, int s, int t0, int L, int ch0, int n, int tid,
                                               int nthreads) {
    const E *x = static_cast<const E *>(cv.x);
    const E *ci = static_cast<const E *>(cv.cs_in);
    E *co = static_cast<E *>(cv.cs_out);
    for (int c = ch0 + tid; c < ch0 + n; c += nthreads) {
        E v[kConvHist];
#pragma unroll
        for (int j = 0; j < kConvHist; ++j) {
            const int pos = L - kConvHist + j;
            v[j] = pos >= 0 ? x[(size_t)(t0 + pos) * cv.conv_dim + c]
                 : ci     ? ci[((size_t)s * kConvHist + (kConvHist + pos)) * cv.conv_dim + c]
                          : E(0);
        }
#pragma unroll
        for (int j = 0; j < kConvHist; ++j) co[((size_t)s * kConvHist + j) * cv.conv_dim + c] = v[j];
    }
}

__device__ __forceinline__ void conv_rows(const ConvOut &cv, int s, int t0, int L, int ch0, int n, int tid,
                                          int nthreads) {
    if (cv.esz == 2) conv_rows_copy<uint16_t>(cv, s, t0, L, ch0, n, tid, nthreads);
    else conv_rows_copy<uint32_t>(cv, s, t0, L, ch0, n, tid, nthreads);
}

// Sequence with chunk-count rank r (rank 0: the most chunks; ties by index) among N <= 64
// sequences: lane i holds sequence i's chunk count and counts the sequences ranked before it.
__device__ __forceinline__ int seq_by_rank(const int32_t *cu, int N, int Ttot, int r) {
    const int lane = threadIdx.x & (kWave - 1);
    const int mine = lane < N ? n_chunks(seq_end(cu, lane, Ttot) - seq_begin(cu, lane)) : -1;
    int ahead = 0;
    for (int j = 0; j < N; ++j) {
        const int other = __shfl(mine, j, kWave);
        ahead += (other > mine || (other == mine && j < lane)) ? 1 : 0;
    }
    const unsigned long long hit = __ballot(lane < N && ahead == r);
    return __builtin_amdgcn_readfirstlane(__ffsll((long long)hit) - 1);
}

// COH: records come from a concurrently running chunk-local kernel (wait for each chunk's
// flag, read device-coherently; the conv cache of the fused prefill is written here, see
// ConvOut); otherwise plain cached reads.
// Gated RMSNorm epilogue in the state pass (NORM instances, D = 128, the concurrent
// schedule's eight-wave workgroups; the layer output of "7.6 Qwen3.5: the linear-attention
// hybrid", section 7.6.2: the core output passes RMSNorm and is gated by SiLU(z), the
// RMSNorm of section 7.6.3 in fp32 with the gain as given).  The compute waves leave each
// chunk's two O strips in LDS instead of storing them; waves 6 and 7, otherwise idle,
// take them, publish each row's sum of squares over the workgroup's 32 columns, combine
// the four workgroups' sums of the row a few steps later and write the normalised, gated
// rows.  o never reaches memory.
constexpr int kNormOst = 36;                        // fp32 row stride of a staged O strip pair
constexpr int kNormBuf = kChunk * kNormOst * 4;     // one chunk's staged strips (bytes)
constexpr int kNormLag = 4;                         // a row sum stored in step j + 1 is loaded in step j + kNormLag

template <int D, bool NORM = false>
constexpr int state_lds_bytes() { return 2 * Rec<D>::U_OFF + (NORM ? 2 * kNormBuf : 0); }

struct StateArgs {
    const char *ws;
    const int32_t *cu;
    int Ttot, Hv, units;
    const float *s0;
    float *sf, *o;
    int ncmax, g0, g1;
    float *mid;
    const flag_t *flags;
    flag_t flag_val;
    ConvOut cv;
    unsigned long long *status;
    int kgroup;   // as in LocalArgs: head h's K^T is in the records of head h - h % kgroup
    // gated RMSNorm epilogue (NORM instances): gate rows z ([T][Hv D] fp16), output rows out
    // ([T][Hv D] bf16), the gain (D, bf16), epsilon, and the row-sum words
    // [Hv][ncmax][D / 32][64] (high half: the call's tag, low half: the fp32 sum)
    const f16 *nz = nullptr;
    const bf16 *ngamma = nullptr;
    bf16 *nout = nullptr;
    float neps = 0.f;
    unsigned long long *nsums = nullptr;
};

// The NW norm waves of one state-pass workgroup (w = 0 .. NW - 1: waves 8 - NW .. 7; wave w
// takes rows 64 w / NW .. of every chunk, NW lanes of 32 / NW columns per row; the workgroup's
// strip pair p holds columns 32 p .. 32 p + 31).  Waves w and w + 4 of a workgroup share a
// SIMD, so waves 6 and 7 (NW = 2) run beside the copy waves; four norm waves, two of them
// beside the compute waves, measured 3 to 4 us slower per call at 4096 tokens x 16 heads.
// They take the compute waves' barriers.  For chunk j:
//  - step j + 1, first thing: its O strips from LDS into registers; each row's sum of
//    squares over the 32 columns goes out as one 64-bit word, the call's tag in the high
//    half and the sum in the low half (a single store: no flag, no wait for completion);
//  - step j + kNormLag: the words of the head's D / 32 workgroups for these rows, and the
//    gates, are loaded;
//  - step j + kNormLag + 2: once every word carries the tag, the sums are added in
//    workgroup order (the same in every workgroup, so results do not depend on timing) and
//    the normalised, gated rows are stored (z fp16, out bf16).
// A word is loaded three steps after it was stored and used two steps after that, so no
// barrier waits on device-coherent traffic unless a workgroup of the head lags (with two
// steps, measured at 4096 tokens x 16 heads, 8 % of the loads still missed a word and the
// waits fed each other); the last chunks are finished after the loop.  A wait that runs out
// (the bound of the record waits) reports GDN_ERR_TIMEOUT and writes NaN.
template <int D, int NW>
__device__ __forceinline__ void norm_waves(const StateArgs &P, const char *obuf, int w, int lane, int pair, int h,
                                           int t0, int L, int c_lo, int c_hi, int gbase, unsigned tag) {
    constexpr int NP = D / 32;          // workgroups per head (strip pairs)
    constexpr int RPW = kChunk / NW;    // rows per wave
    constexpr int LPR = kWave / RPW;    // lanes per row
    constexpr int CPL = 32 / LPR;       // columns per lane
    constexpr int WPL = NP / LPR;       // row-sum words per lane
    static_assert(NP == 4 && (NW == 2 || NW == 4) && CPL % 8 == 0 && WPL >= 1, "norm lane layout");
    const int Hv = P.Hv;
    const int q = lane % LPR;                         // lane in its row
    const int r = RPW * w + lane / LPR;               // row in the chunk
    const int cl = CPL * q;                           // first column in the workgroup's 32
    const int cb = 32 * pair + cl;                    // first column in the head
    const size_t rstride = (size_t)Hv * D;
    float gm[CPL];
#pragma unroll
    for (int i = 0; i < CPL / 8; ++i) {
        const bf16x8 g8 = *reinterpret_cast<const bf16x8 *>(P.ngamma + cb + 8 * i);
#pragma unroll
        for (int e = 0; e < 8; ++e) gm[8 * i + e] = (float)g8[e];
    }
    int spin_max = kSpinMax;
    {
        const unsigned long long sw = __hip_atomic_load(P.status + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((unsigned)(sw >> 32) == kSpinTag) spin_max = (int)(sw & 0x7fffffffu);
    }
    unsigned long long *sums = P.nsums + ((size_t)h * P.ncmax + gbase) * NP * 64;   // chunk c: + c * NP * 64
    auto rows_of = [&](int c) { return min(kChunk, L - c * kChunk); };
    struct Strip { f32x4 v[CPL / 4]; };
    struct Pend {
        unsigned long long wd[WPL];   // the words of workgroups WPL q .. WPL q + WPL - 1
        f16x8 z[CPL / 8];
    };
    // step j + 1: chunk j's strips from LDS (buffer j & 1), row sums out
    auto take = [&](int c, Strip &S_) {
        const float *src = reinterpret_cast<const float *>(obuf + (c & 1) * kNormBuf) + r * kNormOst + cl;
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < CPL / 4; ++i) {
            S_.v[i] = *reinterpret_cast<const f32x4 *>(src + 4 * i);
#pragma unroll
            for (int e = 0; e < 4; ++e) ss = fmaf(S_.v[i][e], S_.v[i][e], ss);
        }
#pragma unroll
        for (int m = 1; m < LPR; m <<= 1) ss += __shfl_xor(ss, m, kWave);   // the same value in every lane of the row
        // every lane of the row stores the same word (no branch around the store)
        __hip_atomic_store(sums + ((size_t)c * NP + pair) * 64 + r,
                           ((unsigned long long)tag << 32) | __builtin_bit_cast(unsigned, ss), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    };
    auto load_words = [&](int c, Pend &Q) {
#pragma unroll
        for (int i = 0; i < WPL; ++i)
            Q.wd[i] = __hip_atomic_load(sums + ((size_t)c * NP + WPL * q + i) * 64 + r, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
    };
    // step j + kNormLag: the words and gates of chunk j (full: all its rows are tokens)
    auto fetch = [&](int c, Pend &Q, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        load_words(c, Q);
        if (FULL || r < rows_of(c)) {
            const f16 *zr = P.nz + (size_t)(t0 + c * kChunk + r) * rstride + (size_t)h * D + cb;
#pragma unroll
            for (int i = 0; i < CPL / 8; ++i) Q.z[i] = *reinterpret_cast<const f16x8 *>(zr + 8 * i);
        } else {
#pragma unroll
            for (int i = 0; i < CPL / 8; ++i) Q.z[i] = f16x8{};
        }
    };
    auto tagged = [&](const Pend &Q) {
        bool ok = true;
#pragma unroll
        for (int i = 0; i < WPL; ++i) ok = ok && (unsigned)(Q.wd[i] >> 32) == tag;
        return __ballot(!ok) == 0;
    };
    // step j + kNormLag + 2: out = o * rsqrt(mean o^2 + eps) * gamma * SiLU(z)
    auto finish = [&](int c, const Strip &S_, Pend &Q, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        bool ok = tagged(Q);
        for (int it = 0; !ok && it < spin_max; ++it) {
            __builtin_amdgcn_s_sleep(2);
            load_words(c, Q);
            ok = tagged(Q);
        }
        if (!ok && lane == 0) report_status(P.status, kStatusTimeout);
        // the NP sums of the row, added in workgroup order (word p sits in lane p / WPL of the row)
        float tot = 0.f;
#pragma unroll
        for (int p = 0; p < NP; ++p)
            tot += __shfl(__builtin_bit_cast(float, (unsigned)Q.wd[p % WPL]), lane - q + p / WPL, kWave);
        const float rn = ok ? rsqrtf(tot * (1.0f / D) + P.neps) : __builtin_nanf("");
        if (FULL || r < rows_of(c)) {
            bf16x8 y[CPL / 8];
#pragma unroll
            for (int k = 0; k < CPL; ++k)
                y[k / 8][k % 8] = (bf16)(S_.v[k / 4][k % 4] * rn * gm[k] * silu((float)Q.z[k / 8][k % 8]));
            bf16 *yr = P.nout + (size_t)(t0 + c * kChunk + r) * rstride + (size_t)h * D + cb;
#pragma unroll
            for (int i = 0; i < CPL / 8; ++i) *reinterpret_cast<bf16x8 *>(yr + 8 * i) = y[i];
        }
    };

    static_assert(kNormLag == 4, "the loop below keeps five strips and two loads in flight");
    __syncthreads();   // the compute waves' barrier after their first loads
    // At the top of step c: s0 .. s4 = strips of chunks c - 2 .. c - 6 (LDS reads, complete);
    // the slot of step c (pa when c - c_lo is even, else pb) holds the words and gates of
    // chunk c - 6, the other one those of chunk c - 5, still in flight.  The loads are never
    // copied (a copy would wait for them), and the steps from c_lo + 6 on, whose chunks are
    // all full, have no memory access behind a branch, so the compiler can count them and
    // waits for each load only where it is used.
    Strip s0, s1, s2, s3, s4;
    Pend pa, pb;
    const std::true_type full{};
    const std::false_type part{};
    // chunk c - 1's strips are taken first (its row sums go out before any wait of the
    // step) and enter s0 only after chunk c - 6 has been finished from s4
    auto shift_in = [&](const Strip &t) {
        s4 = s3;
        s3 = s2;
        s2 = s1;
        s1 = s0;
        s0 = t;
    };
    auto first_step = [&](int c, Pend &pq) {   // c < c_lo + 6: only the actions that exist
        if (c - 1 >= c_lo) {
            Strip t;
            take(c - 1, t);
            shift_in(t);
        }
        if (c - 4 >= c_lo) fetch(c - 4, pq, part);
        __syncthreads();
    };
    auto step = [&](int c, Pend &pq) {         // c >= c_lo + 6: chunks c - 6 and c - 4 are full
        Strip t;
        take(c - 1, t);
        finish(c - 6, s4, pq, full);
        fetch(c - 4, pq, full);
        shift_in(t);
        __syncthreads();
    };
    const int cs = min(c_hi, c_lo + 6);
    for (int c = c_lo; c < cs; ++c) {
        if ((c - c_lo) & 1) first_step(c, pb);
        else first_step(c, pa);
    }
    int c = cs;
    for (; c + 1 < c_hi; c += 2) {   // c - c_lo is even here
        step(c, pa);
        step(c + 1, pb);
    }
    if (c < c_hi) step(c, pa);
    // after the last step: s0 .. s4 = chunks c_hi - 2 .. c_hi - 6; the slot of step c_hi
    // holds chunk c_hi - 6, the other chunk c_hi - 5
    // (the two loaded chunks are finished before the last four are loaded: at most four loads
    // live at once)
    auto tail = [&](Pend &p6, Pend &p5) {
        Strip sl;
        if (c_hi - 1 >= c_lo) take(c_hi - 1, sl);
        if (c_hi - 6 >= c_lo) finish(c_hi - 6, s4, p6, part);
        if (c_hi - 5 >= c_lo) finish(c_hi - 5, s3, p5, part);
        Pend q2, q1;
        if (c_hi - 4 >= c_lo) fetch(c_hi - 4, p6, part);
        if (c_hi - 3 >= c_lo) fetch(c_hi - 3, p5, part);
        if (c_hi - 2 >= c_lo) fetch(c_hi - 2, q2, part);
        if (c_hi - 1 >= c_lo) fetch(c_hi - 1, q1, part);
        if (c_hi - 4 >= c_lo) finish(c_hi - 4, s2, p6, part);
        if (c_hi - 3 >= c_lo) finish(c_hi - 3, s1, p5, part);
        if (c_hi - 2 >= c_lo) finish(c_hi - 2, s0, q2, part);
        if (c_hi - 1 >= c_lo) finish(c_hi - 1, sl, q1, part);
    };
    if ((c_hi - c_lo) & 1) tail(pb, pa);
    else tail(pa, pb);
}

// The state pass of workgroup b (waves 0 .. 3 of the workgroup; further waves only take the
// barriers): lds is the workgroup's LDS (state_lds_bytes), sfail_ one LDS word.
template <int D, bool COH, bool NORM = false>
__device__ __forceinline__ void state_pass_body(char *lds, int *sfail_, int b, const StateArgs &P) {
    static_assert(!NORM || (COH && D == 128), "the norm epilogue runs in the concurrent schedule at D = 128");
    using R = Rec<D>;
    constexpr int NKS = R::NKS, NTD = R::NTD, NS = D / 16, NP = NS / 2;
    constexpr int ABYTES = R::U_OFF;                  // A-operand fragments of one chunk
    static_assert(ABYTES % 2048 == 0, "copy granularity");
    const char *__restrict__ ws = P.ws;
    const int32_t *__restrict__ cu = P.cu;
    const int Ttot = P.Ttot, Hv = P.Hv, units = P.units, ncmax = P.ncmax, g0 = P.g0, g1 = P.g1;
    const float *s0 = P.s0;
    float *sf = P.sf, *__restrict__ o = P.o, *mid = P.mid;
    const flag_t *flags = P.flags;
    const flag_t flag_val = P.flag_val;
    const ConvOut &cv = P.cv;
    unsigned long long *status = P.status;
    // the two A-operand buffers: lds and lds + ABYTES
    auto abuf = [lds](int i) { return lds + (i & 1) * ABYTES; };

    // block -> (unit, strip pair) so that the NP blocks of one unit land on the same XCD
    // (workgroups are dealt to the 8 XCDs in turn).  When a key group's value heads share the
    // K^T records and the units fill whole runs of 8 groups, the units of a group land on one
    // XCD as well, so the group's later heads find its K^T lines in that XCD's L2.
    const int v = 8 * (b / (8 * NP)) + (b % 8);
    const int G = P.kgroup;
    const int u = (G > 1 && units % (8 * G) == 0) ? 8 * G * (v / (8 * G)) + G * (v % 8) + (v / 8) % G : v;
    const int pair = (b / 8) % NP;
    if (u >= units) return;
    // With a few sequences (N <= 64) the units go to the sequences longest first, so the
    // workgroups dispatched last, when there are more than the compute units, have the
    // least work (list scheduling in decreasing order).
    const int nseq = units / Hv, h = u % Hv;
    const int s = (cu && nseq > 1 && nseq <= kWave) ? seq_by_rank(cu, nseq, Ttot, u / Hv) : u / Hv;
    // wave index in a scalar register (the direct-to-LDS base and offset must be uniform)
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool copier = wave >= 2;
    const int l16 = lane & 15, kg = lane >> 4;
    const int j = 2 * pair + (wave & 1);
    const int col = 16 * j + l16;
    // wave-uniform values, kept in scalar registers (buffer resources must be uniform)
    const int t0 = __builtin_amdgcn_readfirstlane(seq_begin(cu, s));
    const int L = __builtin_amdgcn_readfirstlane(seq_end(cu, s, Ttot) - t0);
    const int nc = n_chunks(L);
    const int gbase = __builtin_amdgcn_readfirstlane(chunk_base_wave(cu, s));
    auto rec_of = [&](int c) { return ws + ((size_t)h * ncmax + gbase + c) * R::SIZE; };
    // This launch covers the sequence's chunks whose packed index lies in [g0, g1): local
    // chunks [c_lo, c_hi).  The state enters from the initial state when the range starts
    // the sequence and from `mid` otherwise, and leaves to the final state when the range
    // ends the sequence and to `mid` otherwise.  An empty sequence belongs to the launch
    // whose range starts at 0 (its final state is its initial state).
    const int c_lo = min(max(g0 - gbase, 0), nc), c_hi = min(max(g1 - gbase, 0), nc);
    if (nc > 0 ? c_lo >= c_hi : g0 != 0) return;
    const float *s_in = c_lo == 0 ? s0 : mid;
    float *s_out = c_hi == nc ? sf : mid;
    // set by a copy wave whose wait for a record ran out; read by the compute waves after
    // every chunk barrier
    int &sfail = *sfail_;
    if (threadIdx.x == 0) sfail = 0;
    __syncthreads();

    if (wave >= 4) {
        if constexpr (NORM) {
            if (wave >= 6) {   // the SIMDs of the copy waves
                norm_waves<D, 2>(P, lds + 2 * ABYTES, wave - 6, lane, pair, h, t0, L, c_lo, c_hi, gbase,
                                 (unsigned)(flag_val >> 32) ^ (unsigned)flag_val);
                return;
            }
        }
        // waves past the state pass's four (eight-wave workgroups of the combined kernel): they
        // take the same barriers as the copy waves and nothing else
        __syncthreads();
        for (int c = c_lo; c < c_hi; ++c) __syncthreads();
        return;
    }
    if (copier) {
        // Each copy wave moves half of the A operands with direct-to-LDS buffer loads
        // (lane l of each 16-byte load lands at base + 16 l), then waits for them before
        // the barrier that hands the buffer to the compute waves.
        // (wave 2: -W' and Qt; wave 3: K^T, from the record of the key group's first head)
        const int half = (wave - 2) * (ABYTES / 2);
        static_assert(ABYTES / 2 == R::K_OFF, "the second half is K^T");
        const int hsrc = wave == 3 ? h - h % P.kgroup : h;
        auto stage = [&](int c, char *dst) {
            const __amdgpu_buffer_rsrc_t r = make_rsrc(ws + ((size_t)hsrc * ncmax + gbase + c) * R::SIZE, R::SIZE);
            // the NP workgroups of a head copy the same record at the same time: each starts
            // at its own NP-th of the half, so that at any moment they read different lines
            copy_to_lds<COH ? kCohAux : 0>(r, half, dst + half, ABYTES / 2, lane, pair * (ABYTES / 2 / 1024 / NP));
        };
        // With `flags`, the records are written by a chunk-local kernel running at the same
        // time: wait (bounded) until chunk c's record is published; every record load is then
        // device-coherent.  The copy waves confirm a chunk before the barrier after which the
        // compute waves prefetch its U' and Ol^T strips, i.e. two chunks ahead of the compute.
        // the bound on each wait: the workspace header's second word when it holds kSpinTag
        // in its high half (a caller's setting, for tests), else kSpinMax
        int spin_max = kSpinMax;
        if constexpr (COH) {
            const unsigned long long sw = __hip_atomic_load(status + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if ((unsigned)(sw >> 32) == kSpinTag) spin_max = (int)(sw & 0x7fffffffu);
        }
        auto wait_flag = [&](const flag_t *f) {
            for (int it = 0; it < spin_max; ++it) {
                if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == flag_val) return true;
                __builtin_amdgcn_s_sleep(2);
            }
            return __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == flag_val;
        };
        auto ready = [&](int c) {
            if (sfail) return;   // already failed: its outputs are NaN, no further waits
            if (!wait_flag(flags + (size_t)h * ncmax + gbase + c)) {
                sfail = 1;
                if (lane == 0) report_status(status, kStatusTimeout);
            }
        };
        if constexpr (COH) {
            if (c_lo < c_hi) ready(c_lo);
            if (c_lo + 1 < c_hi) ready(c_lo + 1);
        }
        if (c_lo < c_hi) stage(c_lo, abuf(c_lo));
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        for (int c = c_lo; c < c_hi; ++c) {
            // The flag of chunk c + 2 is loaded before this step's copies are issued and tested
            // after them: its round trip then overlaps the copies instead of following them
            // (the load is unconditional, reading chunk c's flag, known to be set, when there is
            // no chunk c + 2, and the empty asm keeps the test after the copies).
            flag_t published = flag_val;
            if constexpr (COH)
                published = __hip_atomic_load(flags + (size_t)h * ncmax + gbase + (c + 2 < c_hi ? c + 2 : c),
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (c + 1 < c_hi) stage(c + 1, abuf(c + 1));
            if constexpr (COH) {
                asm volatile("" : "+v"(published));
                if (c + 2 < c_hi && published != flag_val) ready(c + 2);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        if constexpr (COH) {
            // Conv cache of sequence s (the concurrent schedule covers whole sequences).  Only
            // a sequence's first chunk reads the input cache, and every chunk of head h has
            // been confirmed above: the v channels of head h are free to overwrite.  The q and
            // k channels of key head h / G are read by the first chunks of all G value heads of
            // the group; the group's first head writes them once the others' are published.
            if (cv.cs_out && pair == 0) {
                const int ct = lane + 64 * (wave - 2);
                conv_rows(cv, s, t0, L, 2 * cv.Hk * cv.dk + h * D, D, ct, 128);
                if (h % cv.G == 0) {
                    bool others_read = true;
                    if (nc > 0 && cv.cs_in == cv.cs_out)
                        for (int hh = h + 1; hh < h + cv.G; ++hh)
                            others_read = wait_flag(flags + (size_t)hh * ncmax + gbase) && others_read;
                    const int kh = h / cv.G;
                    if (others_read) {
                        conv_rows(cv, s, t0, L, kh * cv.dk, cv.dk, ct, 128);
                        conv_rows(cv, s, t0, L, (cv.Hk + kh) * cv.dk, cv.dk, ct, 128);
                    } else if (lane == 0) {   // the input cache may still be read: leave it
                        report_status(status, kStatusTimeout);
                    }
                }
            }
        }
        return;
    }

    f32x4 S[NTD];
    const size_t st_off = ((size_t)s * Hv + h) * D * D;
    if (s_in) {
#pragma unroll
        for (int m = 0; m < NTD; ++m)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) S[m][qq] = s_in[st_off + (size_t)(16 * m + 4 * kg + qq) * D + col];
    } else {
#pragma unroll
        for (int m = 0; m < NTD; ++m) S[m] = zero4();
    }
    // this lane's part of the strip's U and Ol tiles (uniform record base + lane offset),
    // kept packed until the step that uses them
    const int strip_off = (j * 4 * 64 + lane) * 12;
    f32x4 Uf[4], Of[4];
    u32x3 Uh0[4] = {}, Oh0[4] = {};
    float gm = 0.f;
    auto load_strip = [&](const char *rec, u32x3 *U_, u32x3 *O_, float &g_) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            U_[mt] = rec_load12(rec, R::U_OFF + strip_off + mt * 768, COH);
            O_[mt] = rec_load12(rec, R::O_OFF + strip_off + mt * 768, COH);
        }
        // lane-varying address: a vector load (no scalar load shares lgkmcnt with LDS reads)
        g_ = COH ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(rec, 1 << 30),
                                                                                   R::GM_OFF + (lane & 3) * 4, 0,
                                                                                   kCohAux))
                   : *reinterpret_cast<const float *>(rec + R::GM_OFF + (lane & 3) * 4);
    };
    // the query scale of the call (stored in every record), applied to the fp32 outputs
    float osc = 1.f;
    auto load_scale = [&](const char *rec) {
        osc = COH ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(rec, 1 << 30),
                                                                                    R::GM_OFF + 16, 0, kCohAux))
                  : *reinterpret_cast<const float *>(rec + R::GM_OFF + 16);
    };
    if (!COH && c_lo < c_hi) {
        load_strip(rec_of(c_lo), Uh0, Oh0, gm);
        load_scale(rec_of(c_lo));
    }
    // Retire the initial state and strip loads here, once.  Left pending into the loop,
    // the compiler's wait analysis merges them into the loop header and then waits for
    // every outstanding access (the previous chunk's o stores and this chunk's prefetch)
    // before the first MFMA of each chunk.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (COH && c_lo < c_hi) {   // first strips only once the copy waves have confirmed them
        load_strip(rec_of(c_lo), Uh0, Oh0, gm);
        load_scale(rec_of(c_lo));
        __builtin_amdgcn_s_waitcnt(0);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) { Uf[mt] = unpack24(Uh0[mt]); Of[mt] = unpack24(Oh0[mt]); }
    // inf / NaN detection for the outputs and the final state: x * 0 is 0 for every finite x
    // and NaN otherwise, so one FMA per value folds them into a sum that ends non-finite
    // exactly when some value was (reported at the end)
    float nfacc = 0.f;

    // o rows of this lane: row 16 mt + 4 kg + qq of the chunk, column col
    // O^T tiles: lane (kg, l16) holds columns 16 j + 4 kg .. + 3 of output row 16 mt + l16
    const int row_stride = Hv * D;
    const int o_lane = l16 * row_stride + 4 * kg;

    // Fragment groups read from LDS (16 fragments each at D = 128).  Phase 1: the -W
    // fragments of all four row tiles (all k steps), then the Qt fragments.  Phase 2 group p:
    // K^T hi and lo fragments of state row tiles 4p .. 4p + 3 (both k steps).
    constexpr int NG2 = NTD / 4;           // phase 2 groups
    constexpr int GF = 16;                 // fragments per group (both phases, D = 128)
    static_assert(4 * NKS <= GF, "group size");
    auto read_p2 = [&](const char *A, int p, f16x8 *F) {
#pragma unroll
        for (int dm = 0; dm < 4; ++dm)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int m = 4 * p + dm;
                F[dm * 4 + ks] = *reinterpret_cast<const f16x8 *>(A + R::K_OFF + ((m * 2 + ks) * 64 + lane) * 16);
                F[dm * 4 + 2 + ks] =
                    *reinterpret_cast<const f16x8 *>(A + R::K_OFF + (((NTD + m) * 2 + ks) * 64 + lane) * 16);
            }
    };

    // One chunk step.  Every chunk but a sequence's last is full, so the main loop runs
    // LAST = false: its next-chunk prefetch and its 16 o stores are unconditional, and the
    // compiler can wait for the prefetch alone (vmcnt counts the stores issued after it)
    // instead of for every outstanding access.
    auto chunk_step = [&](int c, auto last_tag) {
        constexpr bool LAST = decltype(last_tag)::value;
        const char *A = abuf(c);
        u32x3 Un[4], On[4];
        float gn = 0.f;
        if constexpr (!LAST) load_strip(rec_of(c + 1), Un, On, gn);
        f16x8 Sh[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) Sh[ks] = pack_h(S[2 * ks], S[2 * ks + 1]);

        // ---- Delta' = U' + (-W') S first (four row-tile chains, one MFMA per k step), then
        // O^T = Ol^T + S^T Qt^T (four chains): the bf16 split of Delta' below is independent
        // of the O MFMAs and is scheduled among them, off the path from one state to the next
        f16x8 fr[2][GF];
        auto read_a = [&](const char *A_, int off, f16x8 *F) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    F[mt * NKS + ks] = *reinterpret_cast<const f16x8 *>(A_ + off + ((mt * NKS + ks) * 64 + lane) * 16);
        };
        read_a(A, R::W_OFF, fr[0]);
        f32x4 Dl[4], Ot[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) Dl[mt] = mfma16(fr[0][mt * NKS], Sh[0], Uf[mt]);
        __builtin_amdgcn_sched_barrier(0);
        read_a(A, R::Q_OFF, fr[1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 1; ks < NKS; ++ks)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) Dl[mt] = mfma16(fr[0][mt * NKS + ks], Sh[ks], Dl[mt]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) Ot[mt] = mfma16(Sh[0], fr[1][mt * NKS], Of[mt]);
        __builtin_amdgcn_sched_barrier(0);
        read_p2(A, 0, fr[0]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 1; ks < NKS; ++ks)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) Ot[mt] = mfma16(Sh[ks], fr[1][mt * NKS + ks], Ot[mt]);
        constexpr int P2F = 0;   // phase 2's first fragment group sits in fr[0]

        // ---- S = e^{G_c} S + K^T Delta' with Delta' = diag(e^{G_c - G_t}) Delta; K and
        // Delta' as bf16 hi + lo pairs (the lo x lo term is dropped): one six-MFMA chain
        // per state row tile, four tiles interleaved per group
        bf16x8 Dh[2], Dlo[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const Split8 sp = split_tiles(Dl[2 * ks], Dl[2 * ks + 1]);
            Dh[ks] = sp.hi;
            Dlo[ks] = sp.lo;
        }
        auto kf = [](f16x8 x) { return __builtin_bit_cast(bf16x8, x); };   // K fragments are bf16
#pragma unroll
        for (int p = 0; p < NG2; ++p) {
            const f16x8 *F = fr[(P2F + p) & 1];
            f32x4 a[4];
            a[0] = mfma16(kf(F[0]), Dh[0], S[4 * p] * gm);
            __builtin_amdgcn_sched_barrier(0);
            if (p + 1 < NG2) read_p2(A, p + 1, fr[(P2F + p + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int dm = 1; dm < 4; ++dm) a[dm] = mfma16(kf(F[4 * dm]), Dh[0], S[4 * p + dm] * gm);
#pragma unroll
            for (int dm = 0; dm < 4; ++dm) a[dm] = mfma16(kf(F[4 * dm + 1]), Dh[1], a[dm]);
#pragma unroll
            for (int dm = 0; dm < 4; ++dm) a[dm] = mfma16(kf(F[4 * dm]), Dlo[0], a[dm]);
#pragma unroll
            for (int dm = 0; dm < 4; ++dm) a[dm] = mfma16(kf(F[4 * dm + 1]), Dlo[1], a[dm]);
#pragma unroll
            for (int dm = 0; dm < 4; ++dm) a[dm] = mfma16(kf(F[4 * dm + 2]), Dh[0], a[dm]);
#pragma unroll
            for (int dm = 0; dm < 4; ++dm) a[dm] = mfma16(kf(F[4 * dm + 3]), Dh[1], a[dm]);
#pragma unroll
            for (int dm = 0; dm < 4; ++dm) S[4 * p + dm] = a[dm];
        }

        // ---- this chunk's outputs (times the query scale; NaN once a record wait has run
        // out): uniform row base, per-lane 32-bit offsets
        const int tb = t0 + c * kChunk;
        float *ob = o + ((size_t)tb * Hv + h) * D + 16 * j;
        const int rows = min(kChunk, L - c * kChunk);
        const float oscale = (COH && sfail) ? __builtin_nanf("") : osc;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            Ot[mt] = Ot[mt] * oscale;
            if (!LAST || 16 * mt + l16 < rows) {
#pragma unroll
                for (int e = 0; e < 4; ++e) nfacc = __builtin_fmaf(Ot[mt][e], 0.f, nfacc);
                if constexpr (NORM)   // to the norm waves: row 16 mt + l16, this strip's columns
                    *reinterpret_cast<f32x4 *>(lds + 2 * ABYTES + (c & 1) * kNormBuf +
                                               ((16 * mt + l16) * kNormOst + 16 * (wave & 1) + 4 * kg) * 4) = Ot[mt];
                else
                    *reinterpret_cast<f32x4 *>(ob + o_lane + 16 * mt * row_stride) = Ot[mt];
            }
        }
        __syncthreads();                 // next chunk's A operands are in LDS; buffer c & 1 is free
        if constexpr (!LAST) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) { Uf[mt] = unpack24(Un[mt]); Of[mt] = unpack24(On[mt]); }
            gm = gn;
        }
    };
    for (int c = c_lo; c + 1 < c_hi; ++c) chunk_step(c, std::false_type{});
    if (c_lo < c_hi) chunk_step(c_hi - 1, std::true_type{});

    if (s_out) {
        const bool poison = COH && sfail;
#pragma unroll
        for (int m = 0; m < NTD; ++m)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const float v = poison ? __builtin_nanf("") : S[m][qq];
                nfacc = __builtin_fmaf(v, 0.f, nfacc);
                s_out[st_off + (size_t)(16 * m + 4 * kg + qq) * D + col] = v;
            }
    }
    // inf / NaN in an output or the state (an fp16 operand out of range, non-finite inputs,
    // or the poisoning above): one report per wave
    if (__ballot(!__builtin_isfinite(nfacc)) && lane == 0 && !(COH && sfail)) report_status(status, kStatusNonFinite);
}

template <int D, bool COH>
__global__ __launch_bounds__(256) void state_pass_kernel(StateArgs P) {
    __shared__ __attribute__((aligned(16))) char lds[state_lds_bytes<D>()];
    __shared__ int sfail;
    state_pass_body<D, COH>(lds, &sfail, blockIdx.x, P);
}

// The concurrent schedule in one launch.  Workgroups [0, nslots * Hv) run the chunk-local
// kernel, persistent as (slot, head) = (block mod nslots, block / nslots), and publish each
// record with a flag; workgroups [soff, soff + state blocks) run the state pass (waves 0 .. 3;
// with eight-wave workgroups the other four only take its barriers) and wait for the flags;
// the workgroups in between (to make soff a multiple of 8, so that block - soff and block
// fall on the same XCD) end at once.
// Workgroups are dispatched in index order, so a state-pass workgroup starts only once every
// producer has been dispatched, and producers never wait: every wait ends.
// NORM: the state pass also forms the gated RMSNorm epilogue (norm_waves).
template <int D, bool FUSED, typename TX, typename TW, bool NORM = false>
__global__ __launch_bounds__(LocalShape<D>::THREADS) void prefill_concurrent_kernel(LocalArgs<TX, TW> PL,
                                                                                    StateArgs PS, int soff) {
    constexpr int LB = local_lds_bytes<D, TX, FUSED>(), SB = state_lds_bytes<D, NORM>();
    __shared__ __attribute__((aligned(16))) char lds[LB > SB ? LB : SB];
    __shared__ int word;
    const int b = blockIdx.x;
    if (b >= soff) {
        state_pass_body<D, true, NORM>(lds, &word, b - soff, PS);
    } else if (b < PL.nslots * PL.Hv) {
        chunk_local_body<D, FUSED, TX, TW>(lds, &word, b % PL.nslots, b / PL.nslots, PL);
    }
}

// ============================================================== host side

bool chunked_supported(int dk, int dv) { return dk == dv && (dk == 64 || dk == 128); }

static size_t max_chunks(int T, int N) { return (size_t)(T / kChunk) + (size_t)N; }

// Workspace: the per-(chunk, value head) records, one state per (sequence, value head)
// that carries a sequence from one pipeline segment to the next, and one ready flag per
// (value head, chunk) for the concurrent schedule.
static size_t mid_offset(size_t nc, int Hv, int dk) {
    return nc * (size_t)Hv * (dk == 64 ? (size_t)Rec<64>::SIZE : (size_t)Rec<128>::SIZE);
}
static size_t flags_offset(size_t nc, int N, int Hv, int dk) {
    return mid_offset(nc, Hv, dk) + (size_t)N * Hv * dk * dk * sizeof(float);
}
// The layout above starts kWsHeader bytes into the workspace, after the header (status
// word, wait bound).
size_t chunked_workspace_bytes(int T, int N, int Hv, int dk, int dv) {
    (void)dv;
    const size_t nc = max_chunks(T, N);
    return kWsHeader + flags_offset(nc, N, Hv, dk) + nc * (size_t)Hv * sizeof(flag_t);
}

size_t norm_epi_words(int T, int N, int Hv, int dv) { return max_chunks(T, N) * (size_t)Hv * (dv / 32) * 64; }

// ---- segment pipeline of gdn_chunk_prefill: the packed chunk range is cut into
// segments; the chunk-local kernel of segment k + 1 runs on the caller's stream while
// the state pass of segment k runs on a second stream of the library, ordered by events
// only (no spinning).  Each device gets one such stream (default priority) and a small
// pool of events, created on first use and kept for the life of the process.
constexpr int kMaxSegments = 16;

// Compute units of the current device (cached per device; 0 if unknown).
int device_cus() {
    static std::mutex mu;
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] == 0 && hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus[dev] = 0;
    return cus[dev];
}

// Number of pipeline segments.  The overlap pays only when the state pass is long and
// leaves at least half of the compute units to the chunk-local kernel: otherwise the two
// kernels contend for compute units and memory and the event hops between the streams
// cost more than the overlap hides.  (Measured on MI355X, one gdn_prefill call:
// 4096 tokens x 16 heads, 65 chunks, 64 state workgroups: 170 us unsegmented, 183 us in
// 4 segments; 8 sequences, 606 chunks, 512 state workgroups: 1.14 ms vs 1.24 ms;
// 65536 tokens x 32 heads, 1025 chunks, 128 state workgroups: 4.22 ms vs 3.64 ms, and
// with the kernels as they are now 3.63 ms in 4 segments, 3.48 ms in 8, 3.46 ms in 16:
// one segment per 64 chunks, at most 16.)
static int pipeline_segments(int nc, int state_blocks) {
    const int cus = device_cus();
    if (nc < 256 || cus <= 0 || 2 * state_blocks > cus) return 1;
    return std::min(kMaxSegments, nc / 64);
}

struct PipeRes {
    hipStream_t side = nullptr;
    hipEvent_t ev[kMaxSegments + 1] = {};
    // the caller stream of the last concurrent-schedule call; once calls came from more than
    // one stream (multi), the end of each call's combined kernel
    hipEvent_t last_done = nullptr;
    hipStream_t last_stream = nullptr;
    bool has_last = false, multi = false;
    std::mutex mu;   // one concurrent-schedule launch sequence at a time
    unsigned epoch = 0;   // concurrent-schedule calls so far: the low word of their flag value
    bool ready = false;
};
static std::mutex g_pipe_mu;
static PipeRes g_pipe[64];

static hipError_t pipe_resources(PipeRes **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_pipe_mu);
    PipeRes &r = g_pipe[dev];
    if (!r.ready) {
        e = hipStreamCreateWithFlags(&r.side, hipStreamNonBlocking);
        if (e != hipSuccess) return e;
        for (auto &ev : r.ev) {
            e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
            if (e != hipSuccess) return e;
        }
        e = hipEventCreateWithFlags(&r.last_done, hipEventDisableTiming);
        if (e != hipSuccess) return e;
        r.ready = true;
    }
    *out = &r;
    return hipSuccess;
}

// chunk-local workgroups per value head: one per compute unit of the budget (each holds most
// of the LDS), looping over chunks
static int local_slots(int cus, int nchunks, int Hv) {
    return std::max(1, std::min(nchunks, (cus > 0 ? cus : 256) / Hv));
}

template <typename TX, typename TW>
static LocalArgs<TX, TW> local_args(const PrefillArgs &a, int nc, int g0, int g1, int nslots, flag_t *flags,
                                    flag_t flag_val) {
    LocalArgs<TX, TW> P;
    P.q = a.q; P.k = a.k; P.v = a.v; P.g = a.g; P.beta = a.beta;
    P.cu = a.cu;
    P.N = a.N; P.Ttot = a.T; P.Hk = a.Hk; P.Hv = a.Hv;
    P.scale = a.scale;
    P.ws = (char *)a.ws + kWsHeader;
    P.ncmax = nc; P.g0 = g0; P.g1 = g1; P.nslots = nslots;
    P.x = a.fp ? (const TX *)a.fp->x : nullptr;
    P.conv_w = a.fp ? (const TW *)a.fp->w : nullptr;
    P.cs_in = a.fp ? (const TX *)a.fp->cs_in : nullptr;
    P.l2_eps = a.fp ? a.fp->eps : 0.f;
    P.order = a.order;
    P.flags = flags;
    P.flag_val = flag_val;
    P.kgroup = flags ? 1 : a.Hv / a.Hk;
    return P;
}

template <int D>
static hipError_t launch_local(const PrefillArgs &a, hipStream_t st, int nc, int g0, int g1) {
    if (g1 <= g0 || a.T <= 0) return hipSuccess;
    const int nslots = local_slots(device_cus(), g1 - g0, a.Hv);
    const dim3 grid((unsigned)nslots, a.Hv), block(LocalShape<D>::THREADS);
    if (!a.fp) {
        hipLaunchKernelGGL((chunk_local_kernel<D, false, float>), grid, block, 0, st,
                           local_args<float, float>(a, nc, g0, g1, nslots, nullptr, 0));
    } else if (a.fp->bf16) {
        hipLaunchKernelGGL((chunk_local_kernel<D, true, bf16>), grid, block, 0, st,
                           local_args<bf16, bf16>(a, nc, g0, g1, nslots, nullptr, 0));
    } else if (a.fp->w_bf16) {   // fp32 x and caches, bf16 conv weights (the layer's prefill)
        hipLaunchKernelGGL((chunk_local_kernel<D, true, float, bf16>), grid, block, 0, st,
                           local_args<float, bf16>(a, nc, g0, g1, nslots, nullptr, 0));
    } else {
        hipLaunchKernelGGL((chunk_local_kernel<D, true, float>), grid, block, 0, st,
                           local_args<float, float>(a, nc, g0, g1, nslots, nullptr, 0));
    }
    return hipGetLastError();
}

template <int D>
static int state_blocks(int units) { return 8 * (D / 32) * ((units + 7) / 8); }

template <int D>
static StateArgs state_args(const PrefillArgs &a, int nc, int g0, int g1, const flag_t *flags, flag_t flag_val,
                            const ConvOut &cv) {
    StateArgs P;
    P.ws = (const char *)a.ws + kWsHeader;
    P.cu = a.cu;
    P.Ttot = a.T; P.Hv = a.Hv; P.units = a.N * a.Hv;
    P.s0 = a.s0; P.sf = a.sf; P.o = a.o;
    P.ncmax = nc; P.g0 = g0; P.g1 = g1;
    P.mid = reinterpret_cast<float *>((char *)a.ws + kWsHeader + mid_offset(nc, a.Hv, D));
    P.flags = flags;
    P.flag_val = flag_val;
    P.cv = flags ? cv : ConvOut{};
    P.status = reinterpret_cast<unsigned long long *>(a.ws);
    P.kgroup = flags ? 1 : a.Hv / a.Hk;
    return P;
}

template <int D>
static hipError_t launch_state(const PrefillArgs &a, hipStream_t st, int nc, int g0, int g1,
                               const flag_t *flags = nullptr, flag_t flag_val = 0,
                               const ConvOut &cv = ConvOut{}) {
    const int units = a.N * a.Hv;
    if (units <= 0) return hipSuccess;
    const int blocks = state_blocks<D>(units);
    const StateArgs P = state_args<D>(a, nc, g0, g1, flags, flag_val, cv);
    if (flags)
        hipLaunchKernelGGL((state_pass_kernel<D, true>), dim3(blocks), dim3(256), 0, st, P);
    else
        hipLaunchKernelGGL((state_pass_kernel<D, false>), dim3(blocks), dim3(256), 0, st, P);
    return hipGetLastError();
}

// Clear n ready flags (a captured concurrent-schedule call, before its launch).
__global__ void zero_flags_kernel(flag_t *f, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) f[i] = 0ull;
}

// The combined kernel of the concurrent schedule on `st`: the chunk-local workgroups on the
// compute units the state pass leaves, then the state pass's.
// Whether the concurrent schedule of this call forms the gated RMSNorm epilogue itself: the
// layer's element types (fp32 x, bf16 conv weights) at D = 128.
template <int D>
static bool norm_fused(const PrefillArgs &a) {
    return D == 128 && a.norm && a.fp && !a.fp->bf16 && a.fp->w_bf16;
}

template <int D>
static hipError_t launch_concurrent(const PrefillArgs &a, hipStream_t st, int nc, int cus, int sblocks,
                                    flag_t *flags, flag_t flag_val, const ConvOut &cv) {
    const int nslots = local_slots(cus - sblocks, nc, a.Hv);
    const int soff = (nslots * a.Hv + 7) / 8 * 8;
    const dim3 grid((unsigned)(soff + sblocks)), block(LocalShape<D>::THREADS);
    StateArgs PS = state_args<D>(a, nc, 0, nc, flags, flag_val, cv);
    if constexpr (D == 128) {
        if (norm_fused<D>(a)) {
            PS.nz = static_cast<const f16 *>(a.norm->z);
            PS.ngamma = static_cast<const bf16 *>(a.norm->gamma);
            PS.nout = static_cast<bf16 *>(a.norm->out);
            PS.neps = a.norm->eps;
            PS.nsums = a.norm->sums;
            hipLaunchKernelGGL((prefill_concurrent_kernel<D, true, float, bf16, true>), grid, block, 0, st,
                               local_args<float, bf16>(a, nc, 0, nc, nslots, flags, flag_val), PS, soff);
            const hipError_t e = hipGetLastError();
            if (e == hipSuccess) a.norm->fused = true;
            return e;
        }
    }
    if (!a.fp) {
        hipLaunchKernelGGL((prefill_concurrent_kernel<D, false, float, float>), grid, block, 0, st,
                           local_args<float, float>(a, nc, 0, nc, nslots, flags, flag_val), PS, soff);
    } else if (a.fp->bf16) {
        hipLaunchKernelGGL((prefill_concurrent_kernel<D, true, bf16, bf16>), grid, block, 0, st,
                           local_args<bf16, bf16>(a, nc, 0, nc, nslots, flags, flag_val), PS, soff);
    } else if (a.fp->w_bf16) {
        hipLaunchKernelGGL((prefill_concurrent_kernel<D, true, float, bf16>), grid, block, 0, st,
                           local_args<float, bf16>(a, nc, 0, nc, nslots, flags, flag_val), PS, soff);
    } else {
        hipLaunchKernelGGL((prefill_concurrent_kernel<D, true, float, float>), grid, block, 0, st,
                           local_args<float, float>(a, nc, 0, nc, nslots, flags, flag_val), PS, soff);
    }
    return hipGetLastError();
}

// Concurrent schedule: the state pass occupies at most a quarter of the compute units and the
// chunk-local work has enough chunks to fill the rest for more than one round.  Then both run
// at the same time in one launch (prefill_concurrent_kernel): the chunk-local workgroups (on
// the remaining compute units) publish each record with a flag and the state pass's
// workgroups wait for the flags.  A chunk-local workgroup raises a flag only after all of that
// chunk's loads and stores have completed, and the state pass writes the conv cache once the
// records that read the input cache are published, so the kernel's end orders everything.
// (Measured on MI355X at 4096 tokens x 16 heads: launched as two kernels on two streams, the
// second one started ~5.6 us after the first, and an event recorded on or waited for by the
// caller's stream after a kernel delays the caller's next kernel by 4 to 6 us.)
//   A waiting state pass holds its compute units.  Calls on one stream run one after the
// other.  Once calls have come from more than one stream, every combined kernel records an
// event after it, and a call from another stream than the previous one waits for that event:
// so at most two combined kernels run at the same time (the one before the first change of
// stream, which has no event, and the next), whose state passes hold at most half of the
// compute units.
static bool concurrent_ok(int nc, int Hv, int sblocks, int cus) {
    return cus > 0 && 4 * sblocks <= cus && (long long)nc * Hv >= 2LL * (cus - sblocks);
}

// Fused prefill: conv_state_out after everything that reads conv_state_in (it may alias it).
static hipError_t launch_fused_cs_out(const PrefillArgs &a, hipStream_t st) {
    if (!a.fp || !a.fp->cs_out) return hipSuccess;
    PrepArgs p{a.fp->x, a.fp->w, a.cu, a.N, a.fp->cs_in, a.fp->cs_out, nullptr, nullptr, nullptr,
               a.T, a.Hk, a.Hv, a.dk, a.dv, a.fp->bf16, a.fp->eps};
    return launch_conv_state_out(p, st);
}

template <int D>
static hipError_t launch_chunked_t(const PrefillArgs &a, hipStream_t st, int phases) {
    const int nc = (int)max_chunks(a.T, a.N);
    hipError_t e;
    if (phases != 3) {   // one phase on its own (split-phase entry points)
        if (phases & 1) {
            e = launch_local<D>(a, st, nc, 0, nc);
            if (e != hipSuccess) return e;
            e = launch_fused_cs_out(a, st);
            if (e != hipSuccess) return e;
        }
        if (phases & 2) return launch_state<D>(a, st, nc, 0, nc);
        return hipSuccess;
    }
    const int sblocks = state_blocks<D>(a.N * a.Hv);
    const int cus = device_cus();
    flag_t *flags = reinterpret_cast<flag_t *>((char *)a.ws + kWsHeader + flags_offset(nc, a.N, a.Hv, D));
    ConvOut cv;   // the conv cache, written by the concurrent schedule's state pass
    if (a.fp && a.fp->cs_out) {
        cv.x = a.fp->x;
        cv.cs_in = a.fp->cs_in;
        cv.cs_out = a.fp->cs_out;
        cv.esz = a.fp->bf16 ? 2 : 4;
        cv.conv_dim = 2 * a.Hk * a.dk + a.Hv * a.dv;
        cv.Hk = a.Hk;
        cv.G = a.Hv / a.Hk;
        cv.dk = a.dk;
    }
    // Under stream capture (a HIP graph being recorded) everything goes on `stream` and no
    // event is recorded or waited for: the concurrent schedule as one launch after a kernel
    // that clears its flags (each replay then uses the graph's fixed flag value), otherwise
    // the two phases one after the other (the segmented schedule's second stream cannot be
    // captured as it runs).
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if ((e = hipStreamIsCapturing(st, &cap)) != hipSuccess) return e;
    if (cap != hipStreamCaptureStatusNone) {
        if (concurrent_ok(nc, a.Hv, sblocks, cus)) {
            const int nflags = nc * a.Hv;
            hipLaunchKernelGGL(zero_flags_kernel, dim3((nflags + 255) / 256), dim3(256), 0, st, flags, nflags);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            if (norm_fused<D>(a)) {   // the epilogue's row-sum words as well
                const int nn = nflags * (D / 32) * 64;
                hipLaunchKernelGGL(zero_flags_kernel, dim3((nn + 255) / 256), dim3(256), 0, st, a.norm->sums, nn);
                if ((e = hipGetLastError()) != hipSuccess) return e;
            }
            return launch_concurrent<D>(a, st, nc, cus, sblocks, flags, ((flag_t)kFlagTagGraph << 32) | 1u, cv);
        }
        if ((e = launch_local<D>(a, st, nc, 0, nc)) != hipSuccess) return e;
        if ((e = launch_state<D>(a, st, nc, 0, nc)) != hipSuccess) return e;
        return launch_fused_cs_out(a, st);
    }
    if (concurrent_ok(nc, a.Hv, sblocks, cus)) {
        PipeRes *pr = nullptr;
        if ((e = pipe_resources(&pr)) != hipSuccess) return e;
        std::lock_guard<std::mutex> lock(pr->mu);
        const flag_t flag_val = ((flag_t)kFlagTag << 32) | ++pr->epoch;
        const bool other = pr->has_last && pr->last_stream != st;
        if (other && pr->multi && (e = hipStreamWaitEvent(st, pr->last_done, 0)) != hipSuccess) return e;
        if (other) pr->multi = true;
        if ((e = launch_concurrent<D>(a, st, nc, cus, sblocks, flags, flag_val, cv)) != hipSuccess) return e;
        if (pr->multi && (e = hipEventRecord(pr->last_done, st)) != hipSuccess) return e;
        pr->last_stream = st;
        pr->has_last = true;
        return hipSuccess;
    }
    const int G = pipeline_segments(nc, sblocks);
    if (G == 1) {
        e = launch_local<D>(a, st, nc, 0, nc);
        if (e != hipSuccess) return e;
        e = launch_state<D>(a, st, nc, 0, nc);
        if (e != hipSuccess) return e;
        return launch_fused_cs_out(a, st);
    }
    PipeRes *pr = nullptr;
    e = pipe_resources(&pr);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(pr->mu);
    for (int k = 0; k < G; ++k) {
        const int g0 = (int)((long long)k * nc / G), g1 = (int)((long long)(k + 1) * nc / G);
        if ((e = launch_local<D>(a, st, nc, g0, g1)) != hipSuccess) return e;
        if ((e = hipEventRecord(pr->ev[k], st)) != hipSuccess) return e;
        if ((e = hipStreamWaitEvent(pr->side, pr->ev[k], 0)) != hipSuccess) return e;
        if ((e = launch_state<D>(a, pr->side, nc, g0, g1)) != hipSuccess) return e;
    }
    if ((e = hipEventRecord(pr->ev[kMaxSegments], pr->side)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(st, pr->ev[kMaxSegments], 0)) != hipSuccess) return e;
    return launch_fused_cs_out(a, st);
}

// Read (and with `clear`, reset) the workspace status word once everything a call enqueued
// has completed: the caller's stream and the library's second stream of this device.
hipError_t workspace_status(void *ws, hipStream_t st, unsigned long long *word, bool clear) {
    hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess) return e;
    int dev = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if (dev >= 0 && dev < 64) {
        hipStream_t side = nullptr;
        {
            std::lock_guard<std::mutex> lock(g_pipe_mu);
            if (g_pipe[dev].ready) side = g_pipe[dev].side;
        }
        if (side && (e = hipStreamSynchronize(side)) != hipSuccess) return e;
    }
    if ((e = hipMemcpy(word, ws, sizeof(*word), hipMemcpyDeviceToHost)) != hipSuccess) return e;
    if (clear) {
        const unsigned long long zero = 0;
        e = hipMemcpy(ws, &zero, sizeof(zero), hipMemcpyHostToDevice);
    }
    return e;
}

// cu_seqlens on the host (synchronous; the debug check only).
hipError_t copy_seqlens(const int32_t *cu, int n, hipStream_t st, int32_t *host) {
    hipError_t e = hipMemcpyAsync(host, cu, sizeof(int32_t) * (size_t)n, hipMemcpyDeviceToHost, st);
    if (e != hipSuccess) return e;
    return hipStreamSynchronize(st);
}

hipError_t launch_prefill_chunked(const PrefillArgs &a, hipStream_t st, int phases) {
    switch (a.dk) {
        case 64: return launch_chunked_t<64>(a, st, phases);
        case 128: return launch_chunked_t<128>(a, st, phases);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn

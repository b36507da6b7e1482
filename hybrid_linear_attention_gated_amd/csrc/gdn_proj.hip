// gdn_proj.hip -- the linear-attention layer's projections on bf16 MFMA:
//
//   y[m][n] = sum_k a[m][k] w[n][k]     (w stored as a linear layer stores its weight)
//
// "7.6 Qwen3.5: the linear-attention hybrid", section 7.6.2: a bias-free input
// projection of the layer input gives the pre-conv q|k|v, the output gate z and the
// two gate pre-activations per value head; the gated RMSNorm's output passes a
// bias-free output projection.  The input projection's epilogue splits its columns
// into x (q|k|v: bf16, or fp32 inside the layer calls), z (bf16), g = -softplus(a) and
// beta = sigmoid(b) (fp32): the maps that turn the gate pre-activations into a log-decay
// and an update gate.
//
// Design (dense contraction: MFMA-bound at these shapes, K = 1024 or 2048):
//  - One 256-thread workgroup (4 waves, 2 x 2) per output tile; a wave owns a
//    WM x WN block: WM = WN = 128 (tile 256 x 256, 256 fp32 accumulators per lane in
//    the accumulator registers) when there are enough tiles to fill the chip, else
//    WM = WN = 64 (tile 128 x 128).
//  - 32 x 32 x 16 MFMAs.  The weight rows are the A operand and the activation rows
//    the B operand, so a lane's accumulator holds runs of 4 consecutive output
//    columns of one row: 8-byte stores.  Both operands are k-contiguous rows, so a
//    lane's fragment (8 consecutive k of one row) is one 16-byte LDS read, and one
//    k-step's fragments (8 reads for 16 MFMAs in the large tile) are small enough to
//    double-buffer beside 256 accumulators.
//  - k advances BK at a time (64 for the large tile, 128 for the small one when K
//    allows) through two LDS stages: every thread loads its share of a stage into
//    registers with buffer loads (rows past the matrix edge read as zeros) two stages
//    ahead, in one of two register sets, and writes it to the idle LDS stage during
//    the stage before its use; one barrier per stage orders everything.  The loop body has no branch;
//    the fragments of k-step s + 1 are read from LDS between the MFMAs of step s (one
//    read per group of MFMAs, by scheduling hints), so with one wave per SIMD the
//    matrix unit does not wait on LDS.  The 16-byte chunks of an LDS row are
//    XOR-swizzled by row bits (swz below), so the 16 rows of one fragment read land
//    in the LDS's 16 different 16-byte bank groups.
//  - Tiles are numbered so that each XCD (workgroups are dealt to the eight XCDs in
//    turn) takes a contiguous run of tiles in which groups of four row tiles share
//    column tiles: the tiles resident on one XCD at a time reuse each other's rows
//    from its L2.
//  - The gate columns (2 Hv of them) are left out of the tile grid: before the tiles,
//    workgroups of 16 rows each split k over their four waves, sum the partial
//    products through LDS and apply the gate maps (one 16-column tile per wave).
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

#include <algorithm>

namespace gdn {

constexpr int kProjThreads = 256;
constexpr int kGateRows = 16;        // rows per gate workgroup
constexpr int kGateMaxTiles = 4;     // 16-column tiles of gate outputs: 2 Hv <= 64
constexpr int kGateBatch = 8;        // k-steps per wave whose loads are in flight together
constexpr int kTileGroup = 4;        // row tiles that share a run of column tiles

template <int WM, int WN, int BK>
struct ProjTile {
    static constexpr int BM = 2 * WM, BN = 2 * WN;
    static constexpr int MT = WM / 32, NT = WN / 32;     // 32 x 32 MFMA blocks per wave
    static constexpr int ROWB = BK * 2;                  // LDS bytes per row (one k stage)
    static constexpr int CPR = ROWB / 16;                // 16-byte chunks per row
    static constexpr int RPP = kProjThreads / CPR;       // rows one pass of the threads stages
    static constexpr int A_BYTES = BM * ROWB, W_BYTES = BN * ROWB;
    static constexpr int STAGE = A_BYTES + W_BYTES;
    static constexpr int LDS = 2 * STAGE;
    static constexpr int A_LD = BM / RPP, W_LD = BN / RPP;   // 16-byte chunks per thread and stage
    static constexpr int KSTEPS = BK / 16;               // MFMA k-steps of 16 per stage
    static_assert(LDS >= (kProjThreads / kWave) * kGateMaxTiles * kWave * 16, "gate partial sums fit");
};

typedef float f32x16 __attribute__((ext_vector_type(16)));

// D += A B with A 32 x 16, B 16 x 32 (bf16), D 32 x 32 (fp32): lane l holds
// A[l % 32][8 (l / 32) + v] and B[8 (l / 32) + v][l % 32] for v < 8, and
// D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32] for v < 16.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Byte offset of 16-byte chunk c of LDS row `row`.  The LDS serves a 16-byte access of
// 16 lanes per cycle from its 64 four-byte banks, i.e. sixteen 16-byte bank groups, and
// a fragment read has 16 consecutive rows read at one chunk index.  With 128-byte rows
// two rows fill the 64 banks (even rows the lower half), so the chunk index is XORed
// with bits 1..3 of the row; with 256-byte rows, with bits 0..3.  Either way the 16 rows
// hit 16 different groups, and the staging writes (16 lanes = 16 chunks of one or two
// rows) stay conflict-free.  (An XOR with bits 0..2 alone maps rows r and r + 8 onto the
// same banks: a 2-way conflict on every fragment read.)
template <int ROWB>
__device__ __forceinline__ int swz(int row, int c) {
    static_assert(ROWB == 128 || ROWB == 256, "row of 8 or 16 chunks");
    const int f = ROWB == 128 ? (row >> 1) & 7 : row & 15;
    return row * ROWB + ((c ^ f) << 4);
}

__device__ __forceinline__ bf16x8 zero8() {
    bf16x8 z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (bf16)0.f;
    return z;
}

__device__ __forceinline__ void store_bf16x4(bf16 *p, f32x4 v) {
    bf16x4 o;
    o[0] = (bf16)v[0]; o[1] = (bf16)v[1]; o[2] = (bf16)v[2]; o[3] = (bf16)v[3];
    *reinterpret_cast<bf16x4 *>(p) = o;
}

// log(1 + e^x) in fp32: x itself beyond 20 (e^-20 is below fp32 resolution there),
// else log1p(e^x), accurate also far to the left where it tends to e^x.
__device__ __forceinline__ float softplus_f32(float x) { return x > 20.f ? x : log1pf(expf(x)); }
__device__ __forceinline__ float sigmoid_f32(float x) { return 1.f / (1.f + expf(-x)); }

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over the rows [r0, rows) of a [rows][K] bf16 matrix: loads past the
// last row return zeros (the hardware's range check), which pads the tile edges.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const bf16 *base, int r0, int rows, int K) {
    const long bytes = (long)max(rows - r0, 0) * K * 2;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16 *>(base + (size_t)r0 * K), (short)0,
                                             (int)min(bytes, (long)0x7fffffff), 0x00020000);
}

// Kernel modes: plain (bf16 outputs), the layer's input projection (fp32 x) and the layer
// prefill's input projection (fp32 x, fp16 z).  (Each store kind is its own instance: as a
// run-time branch beside the plain store the fp32 one cost the large tile's epilogue 16
// spilled registers.)
enum { kProjPlain = 0, kProjLayerIn = 1, kProjLayerInZ = 2 };

// z as fp16, clamped to the fp16 range (an out-of-range gate stays finite)
__device__ __forceinline__ void store_f16x4_sat(f16 *p, f32x4 v) {
    f16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (f16)__builtin_fminf(__builtin_fmaxf(v[e], -65504.f), 65504.f);
    *reinterpret_cast<f16x4 *>(p) = o;
}

// Four consecutive outputs y[m][n .. n + 3] (n % 4 == 0, so the four lie on one side of
// n_split, a multiple of 4): columns before n_split to y0 (bf16; fp32 for the layer's input
// projections), the others to y1 (bf16; fp16 for the layer prefill's).
template <int MODE>
__device__ __forceinline__ void store_out(const ProjArgs &p, int m, int n, f32x4 v) {
    if (n < p.n_split) {
        if (MODE != kProjPlain) *reinterpret_cast<f32x4 *>(static_cast<float *>(p.y0) + (size_t)m * p.ld0 + n) = v;
        else store_bf16x4(static_cast<bf16 *>(p.y0) + (size_t)m * p.ld0 + n, v);
        return;
    }
    if (MODE == kProjLayerInZ) store_f16x4_sat(static_cast<f16 *>(p.y1) + (size_t)m * p.ld1 + (n - p.n_split), v);
    else store_bf16x4(static_cast<bf16 *>(p.y1) + (size_t)m * p.ld1 + (n - p.n_split), v);
}

// One output tile: rows m0.., columns n0.. of the main (non-gate) columns.
// k stages [kt0, kt1) of the tile; with p.ksplit > 1 the fp32 sums go to partial sum
// plane `split` instead of the bf16 outputs.
template <int WM, int WN, int BK, int MODE>
__device__ __forceinline__ void proj_tile(const ProjArgs &p, int tm, int tn, char *smem, int kt0, int kt1,
                                          int split) {
    using S = ProjTile<WM, WN, BK>;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = tm * S::BM, n0 = tn * S::BN;
    const int K = p.K, M = p.M, N = p.N;
    const __amdgpu_buffer_rsrc_t ra_src = rows_rsrc(static_cast<const bf16 *>(p.a), m0, M, K);
    const __amdgpu_buffer_rsrc_t rw_src = rows_rsrc(static_cast<const bf16 *>(p.w), n0, N, K);

    // staging: thread tid moves chunk tid % CPR of rows tid / CPR + RPP i; two register
    // sets, so a stage's loads are issued two stages before their LDS writes
    const int crow = tid / S::CPR, cc = tid % S::CPR;
    const int voff = crow * K * 2 + cc * 16;
    struct Stg {
        u32x4 a[S::A_LD], w[S::W_LD];
    };
    auto gload = [&](int kt, Stg &r) {
        const int vo = voff + kt * S::ROWB;
#pragma unroll
        for (int i = 0; i < S::A_LD; ++i) r.a[i] = __builtin_amdgcn_raw_buffer_load_b128(ra_src, vo, i * S::RPP * K * 2, 0);
#pragma unroll
        for (int i = 0; i < S::W_LD; ++i) r.w[i] = __builtin_amdgcn_raw_buffer_load_b128(rw_src, vo, i * S::RPP * K * 2, 0);
    };
    auto swrite = [&](int buf, const Stg &r) {
        char *sa = smem + buf * S::STAGE, *sw = sa + S::A_BYTES;
#pragma unroll
        for (int i = 0; i < S::A_LD; ++i) *reinterpret_cast<u32x4 *>(sa + swz<S::ROWB>(crow + S::RPP * i, cc)) = r.a[i];
#pragma unroll
        for (int i = 0; i < S::W_LD; ++i) *reinterpret_cast<u32x4 *>(sw + swz<S::ROWB>(crow + S::RPP * i, cc)) = r.w[i];
    };

    f32x16 acc[S::NT][S::MT];
#pragma unroll
    for (int i = 0; i < S::NT; ++i)
#pragma unroll
        for (int j = 0; j < S::MT; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int arow = wm * WM + (lane & 31), wrow = wn * WN + (lane & 31);
    // fragments of one k-step of 16: lane holds 8 consecutive k of its row
    struct Frags {
        bf16x8 a[S::MT], w[S::NT];
    };
    auto fread = [&](int buf, int s, Frags &f) {
        const char *sa = smem + buf * S::STAGE, *sw = sa + S::A_BYTES;
        const int c = s * 2 + (lane >> 5);
#pragma unroll
        for (int j = 0; j < S::MT; ++j) f.a[j] = *reinterpret_cast<const bf16x8 *>(sa + swz<S::ROWB>(arow + 32 * j, c));
#pragma unroll
        for (int i = 0; i < S::NT; ++i) f.w[i] = *reinterpret_cast<const bf16x8 *>(sw + swz<S::ROWB>(wrow + 32 * i, c));
    };
    auto mfmas = [&](const Frags &f) {
#pragma unroll
        for (int i = 0; i < S::NT; ++i)
#pragma unroll
            for (int j = 0; j < S::MT; ++j) acc[i][j] = mfma32(f.w[i], f.a[j], acc[i][j]);
    };
    constexpr int FR = S::MT + S::NT;              // fragment reads per k-step
    constexpr int MF = S::MT * S::NT;              // MFMAs per k-step
    constexpr int PER = MF / FR > 0 ? MF / FR : 1; // MFMAs between two reads of the next step

    constexpr int NW = S::A_LD + S::W_LD;          // staging loads (and LDS writes) per stage
    constexpr int W_EACH = NW > MF ? NW / MF : 1;  // LDS writes per group in the last step
    constexpr int M_EACH = MF > NW ? MF / NW : 1;  // MFMAs per group in the last step
    static_assert(MF % FR == 0 || FR % MF == 0, "read / MFMA interleave");
    static_assert((NW > MF ? NW % MF : MF % NW) == 0, "write / MFMA interleave");

    // One stage: `wr` holds stage kt + 1 (loaded a stage ago) and is written to the idle LDS
    // buffer during the last k-step; `ld` (free) receives stage kt + 2's loads at the start.
    // The order is fixed by scheduling groups: step 0's fragment reads, the global loads,
    // each step's MFMAs with the next step's reads between them, the LDS writes between
    // the last step's MFMAs.  Past the end the loads repeat the last stage (never used).
    auto stage = [&](int kt, const Stg &wr, Stg &ld) {
        const int buf = (kt - kt0) & 1;
        Frags f0, f1;
        fread(buf, 0, f0);
        gload(min(kt + 2, kt1 - 1), ld);
#pragma unroll
        for (int s = 0; s < S::KSTEPS; ++s) {
            Frags &cur = (s & 1) ? f1 : f0;
            Frags &nxt = (s & 1) ? f0 : f1;
            if (s + 1 < S::KSTEPS) fread(buf, s + 1, nxt);
            mfmas(cur);
        }
        swrite(buf ^ 1, wr);
        __builtin_amdgcn_sched_group_barrier(0x100, FR, 0);    // DS reads of step 0
        __builtin_amdgcn_sched_group_barrier(0x020, NW, 0);    // VMEM reads of stage kt + 2
#pragma unroll
        for (int s = 0; s + 1 < S::KSTEPS; ++s) {
#pragma unroll
            for (int g = 0; g < FR; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read (step s + 1)
                __builtin_amdgcn_sched_group_barrier(0x008, PER, 0); // MFMA (step s)
            }
        }
#pragma unroll
        for (int g = 0; g < (NW > MF ? MF : NW); ++g) {
            __builtin_amdgcn_sched_group_barrier(0x200, W_EACH, 0);  // DS write (stage kt + 1)
            __builtin_amdgcn_sched_group_barrier(0x008, M_EACH, 0);  // MFMA (last step)
        }
        __syncthreads();
    };
    Stg s0, s1;
    gload(kt0, s0);
    gload(min(kt0 + 1, kt1 - 1), s1);
    swrite(0, s0);
    __syncthreads();
    int kt = kt0;
    for (; kt + 1 < kt1; kt += 2) {
        stage(kt, s1, s0);
        stage(kt + 1, s0, s1);
    }
    if (kt < kt1) stage(kt, s1, s0);

    // lane holds y[m][n + 8 g + 4 (lane / 32) + 0..3] of each 32 x 32 block, g < 4
#pragma unroll
    for (int j = 0; j < S::MT; ++j) {
        const int m = m0 + wm * WM + 32 * j + (lane & 31);
        if (m >= M) continue;
#pragma unroll
        for (int i = 0; i < S::NT; ++i) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * WN + 32 * i + 8 * g + 4 * (lane >> 5);
                if (n >= N) continue;
                if (p.ksplit > 1) {
                    *reinterpret_cast<f32x4 *>(p.partial + ((size_t)split * M + m) * N + n) =
                        f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                    continue;
                }
                store_out<MODE>(p, m, n, f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1],
                                                               acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]});
            }
        }
    }
}

// Gate outputs of rows r0 .. r0 + 15: the 2 Hv gate rows of w start at row N.  Wave
// `wave` takes the k-steps wave, wave + 4, ... (all its loads in flight together, rows
// and gate columns past the edge reading as zeros); the partial sums meet in LDS, and
// wave i finishes gate column tile i (-softplus for the a columns, sigmoid for b).
__device__ __forceinline__ void gate_rows(const ProjArgs &p, int gb, char *smem) {
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int r0 = gb * kGateRows, K = p.K, KS = K / 32, G = 2 * p.heads;
    const int kc = 8 * (lane >> 4);
    const __amdgpu_buffer_rsrc_t ra_src = rows_rsrc(static_cast<const bf16 *>(p.a), r0, p.M, K);
    const __amdgpu_buffer_rsrc_t rw_src = rows_rsrc(static_cast<const bf16 *>(p.w), p.N, p.N + G, K);
    const int voff = (lane & 15) * K * 2 + kc * 2;
    f32x4 acc[kGateMaxTiles];
#pragma unroll
    for (int i = 0; i < kGateMaxTiles; ++i) acc[i] = zero4();
    for (int base = 0; base < KS; base += 4 * kGateBatch) {
        u32x4 af[kGateBatch], wf[kGateBatch][kGateMaxTiles];
#pragma unroll
        for (int b = 0; b < kGateBatch; ++b) {
            // k-steps past K read beyond every row's end: redirect them to k-step 0 with a
            // zero operand instead (a row's bytes stay in range)
            const int ks = base + wave + 4 * b;
            const int kb = ks < KS ? ks * 64 : 0;
            af[b] = __builtin_amdgcn_raw_buffer_load_b128(ra_src, voff + kb, 0, 0);
#pragma unroll
            for (int i = 0; i < kGateMaxTiles; ++i)
                wf[b][i] = __builtin_amdgcn_raw_buffer_load_b128(rw_src, voff + kb, 16 * i * K * 2, 0);
        }
#pragma unroll
        for (int b = 0; b < kGateBatch; ++b) {
            if (base + wave + 4 * b >= KS) continue;
#pragma unroll
            for (int i = 0; i < kGateMaxTiles; ++i)
                acc[i] = mfma16(__builtin_bit_cast(bf16x8, wf[b][i]), __builtin_bit_cast(bf16x8, af[b]), acc[i]);
        }
    }
    f32x4 *part = reinterpret_cast<f32x4 *>(smem);
#pragma unroll
    for (int i = 0; i < kGateMaxTiles; ++i) part[(wave * kGateMaxTiles + i) * kWave + lane] = acc[i];
    __syncthreads();
    // wave i sums tile i over the four waves: lane holds rows r0 + lane % 16, gate
    // columns 16 i + 4 (lane / 16) + 0..3
    const int i = wave, m = r0 + (lane & 15);
    if (i >= kGateMaxTiles || m >= p.M) return;
    f32x4 t = part[i * kWave + lane];
#pragma unroll
    for (int v = 1; v < kProjThreads / kWave; ++v) t += part[(v * kGateMaxTiles + i) * kWave + lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int gi = 16 * i + 4 * (lane >> 4) + r;
        if (gi < p.heads) p.g[(size_t)m * p.heads + gi] = -softplus_f32(t[r]);
        else if (gi < G) p.beta[(size_t)m * p.heads + (gi - p.heads)] = sigmoid_f32(t[r]);
    }
}

template <int WM, int WN, int BK, int MODE>
__global__ __launch_bounds__(kProjThreads) void proj_kernel(ProjArgs p) {
    using S = ProjTile<WM, WN, BK>;
    __shared__ __attribute__((aligned(16))) char smem[S::LDS];
    // the gate workgroups come first: short, they delay every compute unit's first tile
    // by the same small amount instead of forming a tail round after the tiles
    int b = blockIdx.x;
    const int gate_blocks = p.heads > 0 ? (p.M + kGateRows - 1) / kGateRows : 0;
    if (b < gate_blocks) {
        gate_rows(p, b, smem);
        return;
    }
    b -= gate_blocks;
    const int KT = p.K / BK;
    if (p.ksplit > 1) {   // split k: block = (tile, k slice), the slices of a tile adjacent
        const int split = b % p.ksplit, tile = b / p.ksplit, per = KT / p.ksplit;
        proj_tile<WM, WN, BK, MODE>(p, tile / p.tiles_n, tile % p.tiles_n, smem, split * per, split * per + per,
                                    split);
        return;
    }
    // XCD x (blocks x, x + 8, ...) takes tiles [x T / 8, (x + 1) T / 8)
    if ((p.ntiles & 7) == 0) b = (b & 7) * (p.ntiles >> 3) + (b >> 3);
    // groups of kTileGroup row tiles run over all column tiles, row tile fastest
    const int per_group = kTileGroup * p.tiles_n;
    const int grp = b / per_group, first = grp * kTileGroup;
    const int gm = min(kTileGroup, p.tiles_m - first);
    const int r = b - grp * per_group;
    proj_tile<WM, WN, BK, MODE>(p, first + r % gm, r / gm, smem, 0, KT, 0);
}

// Split-k second pass: y = bf16(sum of the ksplit fp32 partial planes, in plane order),
// routed like the tile epilogue; one thread per 4 consecutive columns.
__global__ __launch_bounds__(256) void proj_reduce_kernel(ProjArgs p) {
    const long q = (long)blockIdx.x * 256 + threadIdx.x;
    const int nq = p.N / 4;
    if (q >= (long)p.M * nq) return;
    const int m = (int)(q / nq), n = 4 * (int)(q % nq);
    const size_t plane = (size_t)p.M * p.N, at = (size_t)m * p.N + n;
    f32x4 t = *reinterpret_cast<const f32x4 *>(p.partial + at);
    for (int sp = 1; sp < p.ksplit; ++sp) t += *reinterpret_cast<const f32x4 *>(p.partial + sp * plane + at);
    if (p.y1_f16) store_out<kProjLayerInZ>(p, m, n, t);
    else if (p.y0_f32) store_out<kProjLayerIn>(p, m, n, t);
    else store_out<kProjPlain>(p, m, n, t);
}

template <int WM, int WN, int BK, int MODE>
static hipError_t launch_proj_t(ProjArgs p, hipStream_t st) {
    using S = ProjTile<WM, WN, BK>;
    p.tiles_m = (p.M + S::BM - 1) / S::BM;
    p.tiles_n = (p.N + S::BN - 1) / S::BN;
    p.ntiles = p.tiles_m * p.tiles_n;
    // Split k when the tiles fill a quarter of the compute units or less and a partial-sum
    // buffer is given: the largest divisor of the stage count up to cus / tiles (at least 4)
    // whose planes fit the buffer.  The slices' fp32 sums meet in a second pass, in a fixed
    // order.
    p.ksplit = 1;
    if (p.partial && p.heads == 0) {
        const int KT = p.K / BK, cus = device_cus() > 0 ? device_cus() : 256;
        const int want = cus / p.ntiles;
        for (int d = std::min(want, KT); d >= 4; --d)
            if (KT % d == 0 && (size_t)d * p.M * p.N <= p.partial_cap) {
                p.ksplit = d;
                break;
            }
    }
    const int gate_blocks = p.heads > 0 ? (p.M + kGateRows - 1) / kGateRows : 0;
    const long blocks = (long)p.ntiles * p.ksplit + gate_blocks;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((proj_kernel<WM, WN, BK, MODE>), dim3((unsigned)blocks), dim3(kProjThreads), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.ksplit == 1) return e;
    const long quads = (long)p.M * (p.N / 4);
    hipLaunchKernelGGL(proj_reduce_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, st, p);
    return hipGetLastError();
}

bool proj_gates_supported(int heads) { return 2 * heads <= 16 * kGateMaxTiles; }

template <int MODE>
static hipError_t launch_proj_m(const ProjArgs &a, hipStream_t st) {
    // large tiles when they alone fill the compute units
    const long big = (long)((a.M + 255) / 256) * ((a.N + 255) / 256);
    const int cus = device_cus();
    if (big >= (cus > 0 ? cus : 256)) return launch_proj_t<128, 128, 64, MODE>(a, st);
    // small tiles take k 128 deep per stage when K allows, so a stage's MFMAs outlast its loads
    return a.K % 128 == 0 ? launch_proj_t<64, 64, 128, MODE>(a, st) : launch_proj_t<64, 64, 64, MODE>(a, st);
}

hipError_t launch_proj(const ProjArgs &a, hipStream_t st) {
    if (a.M <= 0) return hipSuccess;
    if (a.y1_f16) return launch_proj_m<kProjLayerInZ>(a, st);
    return a.y0_f32 ? launch_proj_m<kProjLayerIn>(a, st) : launch_proj_m<kProjPlain>(a, st);
}

}  // namespace gdn

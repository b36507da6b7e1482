/*
 * gdn.h -- C ABI of the Gated DeltaNet token-mixer library for AMD MI355X (gfx950).
 *
 * The library computes the linear-attention core of a hybrid model's
 * "linear_attention" layers: a depthwise causal conv1d (kernel 4) + SiLU over
 * the mixed q|k|v projection, L2 normalisation of q and k, and the gated delta
 * rule over a fixed-size per-head state,
 *
 *     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t,
 *
 * computed step by step (decay, retrieve, correct, write, read) as in the
 * recurrent-mode GatedDeltaNet formula of "Hugging Face Transformers:
 * Qwen3.5-MoE series explained", section 4.3, and in "7.6 Qwen3.5: the
 * linear-attention hybrid" (LLM full-stack book), section 7.6.2.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers named as tensors are DEVICE pointers on the current HIP device,
 *    row-major and contiguous.  The caller owns every buffer; the library keeps
 *    no pointer after a call returns and allocates no device memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  All
 *    work is enqueued asynchronously on it; buffers must stay valid until the
 *    stream work completes.  gdn_chunk_prefill with GDN_MATH_MFMA and gdn_prefill
 *    may run part of their work on a second stream of the library (the segmented
 *    schedule below; created once per device, default priority, kept with a few
 *    events for the life of the process); that work's
 *    memory accesses are ordered after everything enqueued on `stream` before the
 *    call and before everything enqueued on it after the call, so to the caller it
 *    behaves as if it ran on `stream`.  Concurrent calls on one device must use
 *    distinct workspaces, as always.
 *  - Element type `dtype` (gdn_conv_qk_prep, gdn_decode_step, ...) is the type of the
 *    pre-conv input x, the conv weights and the conv caches (and of the gate, gain
 *    and output of the gated RMSNorm): GDN_BF16 or GDN_F32.  Everything computed is
 *    fp32: q, k, v, o, g, beta and the recurrent states.
 *    (The outputs of this layer are heavy tailed -- the largest |o| is tens of
 *    times its RMS -- so a 16-bit q / k / v / o tensor alone would cost more than
 *    the 2e-2 RMS-relative accuracy the layer is held to.)
 *  - g is the log of the decay gate (a = exp(g), g <= 0); beta is the update gate.
 *  - Heads: Hk key heads, Hv value heads, Hv % Hk == 0; value head h reads key
 *    head h / (Hv / Hk).  conv_dim = 2*Hk*dk + Hv*dv with channel order q | k | v.
 *  - The recurrent state is key-major: state[n][h][i][j], i < dk, j < dv, i.e.
 *    the transpose of S_t above; outputs are identical.
 *  - cu_seqlens (int32, N+1 entries, cu[0] = 0, non-decreasing, cu[N] = T) packs
 *    N variable-length sequences along T.  NULL means one sequence of length T
 *    (N must then be 1).  Zero-length sequences are allowed.  These device values
 *    are a precondition and are not validated, unless the environment variable
 *    GDN_DEBUG_CHECK is set (to anything but "0") when the library first looks: the
 *    prefill calls then copy cu_seqlens to the host and return GDN_ERR_BAD_SHAPE for a
 *    bad one before launching anything, and wait for their own completion to return
 *    the workspace status (GDN_ERR_TIMEOUT, GDN_ERR_NONFINITE; see
 *    gdn_prefill_workspace_status).  Debug-checked calls synchronise the stream.
 *  - Tensor pointers may be NULL when the tensor is empty (T = 0, or B = 0).
 *  - Every non-NULL device pointer (tensors, cu_seqlens, workspace) must be 16-byte
 *    aligned, as every device allocator returns them: the kernels move 16-byte
 *    vectors and stage rows with 16-byte direct-to-LDS loads.  A misaligned pointer
 *    returns GDN_ERR_ALIGN.
 *  - Size limits (GDN_ERR_BAD_SHAPE beyond them), which keep every byte count the
 *    library forms within 64 bits: Hk, Hv <= 4096; N sequences and B decode rows
 *    <= 2^24; rows of gdn_gated_rmsnorm <= 2^40.
 *  - Return value: GDN_OK or a gdn_status code.  Argument errors are detected on
 *    the host before anything is enqueued; nothing is written then.  Launch
 *    failures map to GDN_ERR_HIP.  No function aborts or throws.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 6

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL_POINTER = 1,   /* a required pointer is NULL                         */
    GDN_ERR_BAD_SHAPE = 2,      /* negative size, Hv % Hk != 0, N inconsistent, ...     */
    GDN_ERR_UNSUPPORTED = 3,    /* head dim / dtype combination not implemented         */
    GDN_ERR_WORKSPACE = 4,      /* workspace NULL or smaller than the queried size      */
    GDN_ERR_HIP = 5,            /* a HIP launch or runtime call failed                  */
    GDN_ERR_ALIAS = 6,          /* an output overlaps an input it must not overlap      */
    GDN_ERR_ALIGN = 7,          /* a device pointer is not 16-byte aligned              */
    GDN_ERR_TIMEOUT = 8,        /* the state pass stopped waiting for a chunk's record  */
    GDN_ERR_NONFINITE = 9       /* a prefill output or final state is inf or NaN        */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Arithmetic of gdn_chunk_prefill.
 *  GDN_MATH_F32        : token-by-token recurrence in fp32 (any dk, dv in {16, 32, 64, 128}).
 *  GDN_MATH_MFMA       : chunked WY / UT form (chunk 64) on 16-bit MFMA with split
 *                        operands where the accuracy needs them (dk = dv in {64, 128});
 *                        about 1e-3 RMS-relative on the 0.8B layer shape.
 *  GDN_MATH_F32_CHUNKED: the same chunked WY / UT form with every product an fp32 sum
 *                        (dk, dv in {16, 32, 64}; one workgroup per (sequence, value head)
 *                        carries the state through the chunks); no workspace. */
typedef enum { GDN_MATH_F32 = 0, GDN_MATH_MFMA = 1, GDN_MATH_F32_CHUNKED = 2 } gdn_math;

/* Order of decay and retrieval in one step of the recurrence (argument `order`).
 *  GDN_ORDER_DECAY_FIRST   : S <- a S; m = S^T k; delta = b (v - m); S += k delta^T;
 *                            o = S^T q ("Hugging Face Transformers: Qwen3.5-MoE series
 *                            explained", section 4.3).  The default.
 *  GDN_ORDER_RETRIEVE_FIRST: m = S^T k from the state before the decay, then
 *                            S <- a S + k [b (v - m)]^T; o = S^T q ("7.6 Qwen3.5: the
 *                            linear-attention hybrid", section 7.6.2, as printed).
 * The pages disagree; the two agree when a = 1.  Any other value ->
 * GDN_ERR_UNSUPPORTED. */
typedef enum { GDN_ORDER_DECAY_FIRST = 0, GDN_ORDER_RETRIEVE_FIRST = 1 } gdn_order;

/*
 * gdn_conv_qk_prep -- depthwise causal conv1d (kernel 4, no bias) + SiLU + split
 * + per-head L2 normalisation of q and k.
 * Source: "7.6 Qwen3.5: the linear-attention hybrid", section 7.6.2 (conv over
 * conv_dim = 2*key_dim + value_dim channels, one filter per channel, left
 * context only; q and k L2-normalised before the recurrence); conv cache per
 * "Hugging Face Transformers: Qwen3.5-MoE series explained", section 8.2.
 *
 *   x              [T][conv_dim]        pre-conv mixed q|k|v
 *   conv_w         [conv_dim][4]        tap 3 multiplies the current token
 *   cu_seqlens     [N+1] or NULL
 *   conv_state_in  [N][3][conv_dim] or NULL (zero history); slot 0 is the oldest
 *   conv_state_out [N][3][conv_dim] or NULL; receives the last three inputs of
 *                  each sequence (reaching into conv_state_in for sequences
 *                  shorter than three).  May alias conv_state_in exactly.
 *   q, k           [T][Hk][dk] fp32     q / sqrt(|q|^2 + l2_eps), same for k
 *   v              [T][Hv][dv] fp32     SiLU(conv) of the value channels
 * y[t][c] = sum_j conv_w[c][j] * x[t-3+j][c] with history from conv_state_in,
 * never crossing a sequence boundary.  dk, dv must be multiples of 8 and <= 256.
 */
int gdn_conv_qk_prep(const void *x, const void *conv_w,
                     const int32_t *cu_seqlens, int N,
                     const void *conv_state_in, void *conv_state_out,
                     float *q, float *k, float *v,
                     int T, int Hk, int Hv, int dk, int dv, int dtype,
                     float l2_eps, void *stream);

/*
 * Workspace bytes gdn_chunk_prefill needs for these sizes and `math` (0 when
 * none is needed).  Upper bound valid for any cu_seqlens with the given T and N.
 */
size_t gdn_chunk_prefill_workspace_size(int T, int N, int Hk, int Hv, int dk, int dv, int math);

/*
 * gdn_chunk_prefill -- gated delta rule over packed sequences, returning the
 * per-token outputs and the final state of each sequence (the chunk-mode call
 * of the prefill path in "Hugging Face Transformers: Qwen3.5-MoE series
 * explained", section 8.2, which returns the output and the last recurrent state).
 *
 *   q, k           [T][Hk][dk] fp32 (L2-normalised by the caller or by gdn_conv_qk_prep)
 *   v              [T][Hv][dv] fp32
 *   g, beta        [T][Hv] fp32
 *   cu_seqlens     [N+1] or NULL
 *   initial_state  [N][Hv][dk][dv] fp32 or NULL (zero state)
 *   final_state    [N][Hv][dk][dv] fp32 or NULL; may alias initial_state exactly
 *   o              [T][Hv][dv]   fp32; o_t = S_t (scale * q_t); must not overlap any input
 *   workspace      device scratch of at least gdn_chunk_prefill_workspace_size()
 *                  bytes (may be NULL when that size is 0); contents are scratch.
 *                  With GDN_MATH_MFMA it starts with a 256-byte header (a status word,
 *                  see gdn_prefill_workspace_status; then an optional bound on the state
 *                  pass's waits, below) and holds the per-(chunk, value head) results of
 *                  the chunk-local phase, one state per (sequence, value head) and one
 *                  ready flag per (chunk, value head).  It needs no initialisation:
 *                  each call's ready flags carry a value of that call's own.
 *   math           gdn_math; GDN_MATH_MFMA or GDN_MATH_F32_CHUNKED with other head dims
 *                  -> GDN_ERR_UNSUPPORTED
 *   order          gdn_order (decay before or after the retrieval)
 *
 * With GDN_MATH_MFMA the two phases below run in one of three schedules, all
 * bit-identical to running the two phases one after the other:
 *  - concurrent, when the state pass occupies at most a quarter of the device's
 *    compute units and there are at least twice as many (chunk, value head) items
 *    as the other compute units: both phases in one launch on `stream`, whose first
 *    workgroups run the chunk-local phase on the compute units the state pass leaves
 *    free and raise a flag in the workspace as each record is complete, while its
 *    last workgroups run the state pass and wait for each flag.  The wait is bounded
 *    (about a second; the header's second 64-bit word, when it holds 0x7370696e in
 *    its high half, sets the bound to its low half in iterations of a ~128-cycle
 *    sleep, for tests): a record that is never published ends the call with NaN
 *    outputs and final states and the status GDN_ERR_TIMEOUT, never in a hang; the
 *    chunk-local phase publishes every record.  Once calls have come from more than
 *    one caller stream, a call from another stream than the previous concurrent one
 *    first waits for that call's launch, so at most two such launches run at a time;
 *  - segmented, when the packed chunks are many (at least 256) and the state pass
 *    occupies at most half of the compute units: the chunks are cut into up to sixteen
 *    segments, and the chunk-local phase of segment k + 1 (on `stream`) runs while
 *    the state pass of segment k runs on the second stream; a sequence's state
 *    passes between segments through the workspace;
 *  - sequential otherwise: both phases on `stream`, one after the other.
 * While `stream` is capturing a HIP graph, the concurrent schedule is captured as a kernel
 * that clears the ready flags followed by the one launch (every replay waits for a
 * graph-only flag value), and the segmented one as the sequential schedule; nothing is
 * enqueued on the library's second stream and no event is recorded or waited for.
 * The query scale multiplies the fp32 outputs after the 16-bit products, so any finite
 * scale is exact to apply; the state pass rounds the state to fp16 for its products,
 * so a state element beyond +-65504 makes outputs non-finite, which the status word
 * reports (GDN_ERR_NONFINITE).
 */
int gdn_chunk_prefill(const float *q, const float *k, const float *v,
                      const float *g, const float *beta,
                      const int32_t *cu_seqlens, int N,
                      const float *initial_state, float *final_state,
                      float *o, float scale,
                      int T, int Hk, int Hv, int dk, int dv, int math, int order,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * The two phases of gdn_chunk_prefill with GDN_MATH_MFMA, for callers that
 * schedule them separately (for example to overlap the parallel chunk-local
 * phase of one layer with other work).  gdn_chunk_prefill_local computes the
 * per-chunk quantities of the chunk form (W, U, the decay-weighted query, the
 * intra-chunk outputs) into `workspace`; gdn_chunk_prefill_state then runs the
 * sequential pass over chunks that carries the state, writes o and the final
 * state.  Arguments mean what they mean for gdn_chunk_prefill; the workspace
 * must not be modified between the two calls, and cu_seqlens, N, T and the head
 * sizes must be the same in both.  Running local then state equals one
 * gdn_chunk_prefill call with GDN_MATH_MFMA.  `order` only enters the local phase.
 */
int gdn_chunk_prefill_local(const float *q, const float *k, const float *v,
                            const float *g, const float *beta,
                            const int32_t *cu_seqlens, int N, float scale,
                            int T, int Hk, int Hv, int dk, int dv, int order,
                            void *workspace, size_t workspace_bytes, void *stream);
int gdn_chunk_prefill_state(const int32_t *cu_seqlens, int N,
                            const float *initial_state, float *final_state, float *o,
                            int T, int Hk, int Hv, int dk, int dv,
                            const void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_prefill -- gdn_conv_qk_prep and gdn_chunk_prefill (GDN_MATH_MFMA) in one call,
 * with the conv prep fused into the chunk-local phase: q, k and v are formed in
 * on-chip memory for each chunk and never written to HBM.  The conv + SiLU + L2 is
 * that of gdn_conv_qk_prep ("7.6 Qwen3.5: the linear-attention hybrid", section
 * 7.6.2) and the recurrence that of gdn_chunk_prefill ("Hugging Face Transformers:
 * Qwen3.5-MoE series explained", sections 4.3 and 8.2).
 *
 *   x, conv_w, conv_state_in, conv_state_out, dtype, l2_eps   as in gdn_conv_qk_prep
 *                  (conv_state_out may alias conv_state_in exactly, or be NULL)
 *   g, beta, initial_state, final_state, o, scale, order   as in gdn_chunk_prefill
 *   dk = dv in {64, 128} (GDN_ERR_UNSUPPORTED otherwise)
 *   workspace      at least gdn_chunk_prefill_workspace_size(T, N, Hk, Hv, dk, dv,
 *                  GDN_MATH_MFMA) bytes; must not overlap any other argument.
 * o, final_state and conv_state_out must not overlap any input except the exact
 * aliases named above.  Errors as for the two calls it replaces.  The schedules are
 * those of gdn_chunk_prefill; in the concurrent one the state pass also writes
 * conv_state_out (after the chunks that read conv_state_in have published), so that
 * nothing follows the state pass on `stream`.
 */
int gdn_prefill(const void *x, const void *conv_w, const int32_t *cu_seqlens, int N,
                const void *conv_state_in, void *conv_state_out,
                const float *g, const float *beta,
                const float *initial_state, float *final_state, float *o,
                float scale, float l2_eps,
                int T, int Hk, int Hv, int dk, int dv, int dtype, int order,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_prefill_workspace_status -- the outcome of the chunked prefills (gdn_chunk_prefill
 * with GDN_MATH_MFMA, the split phases, gdn_prefill, gdn_layer_prefill, whose workspace
 * starts with its prefill's) that used `workspace` since the previous query.  Waits for
 * `stream` and the library's second stream on the current device, reads the status word
 * at the start of the workspace and clears it.
 *   GDN_OK             no failure recorded (or a word that no kernel wrote)
 *   GDN_ERR_TIMEOUT    a state pass stopped waiting for a record, or (the layer prefill's
 *                      norm formed in the state pass) for a row sum (outputs NaN)
 *   GDN_ERR_NONFINITE  an output or a final state came out inf or NaN
 *   GDN_ERR_NULL_POINTER / GDN_ERR_ALIGN / GDN_ERR_WORKSPACE (fewer than 256 bytes),
 *   GDN_ERR_HIP        argument or runtime errors of the query itself
 * A freshly allocated workspace reports GDN_OK unless its first 8 bytes happen to hold
 * the status tag 0x67646e73 in their high half; a caller that wants certainty queries
 * once before the first call.
 */
int gdn_prefill_workspace_status(void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_prefill_local -- the first phase of gdn_prefill: conv prep + chunk-local
 * quantities into `workspace` (and conv_state_out, written after the phase has
 * read conv_state_in), for callers that schedule the phases separately.
 * gdn_chunk_prefill_state then consumes the workspace exactly as after
 * gdn_chunk_prefill_local; the two together equal one gdn_prefill call.
 * Arguments mean what they mean for gdn_prefill.
 */
int gdn_prefill_local(const void *x, const void *conv_w, const int32_t *cu_seqlens, int N,
                      const void *conv_state_in, void *conv_state_out,
                      const float *g, const float *beta, float scale, float l2_eps,
                      int T, int Hk, int Hv, int dk, int dv, int dtype, int order,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_decode_step -- one token for each of B sequences: advance the conv cache by
 * one input, conv + SiLU + L2 on the window, one step of the recurrence on the
 * state, in place (the decode branch of "Hugging Face Transformers: Qwen3.5-MoE
 * series explained", section 8.2: conv-cache update followed by the recurrent
 * rule, both caches written back).
 *
 *   x           [B][conv_dim]       the new token's pre-conv mixed q|k|v
 *   conv_w      [conv_dim][4]
 *   conv_state  [B][3][conv_dim]    in/out: window = [slot0, slot1, slot2, x];
 *                                   afterwards [slot1, slot2, x]
 *   g, beta     [B][Hv] fp32
 *   state       [B][Hv][dk][dv]     fp32, in/out
 *   o           [B][Hv][dv]         fp32; must not overlap any other argument
 *   order       gdn_order, as in gdn_chunk_prefill
 * dk, dv in {16, 32, 64, 128}.
 */
int gdn_decode_step(const void *x, const void *conv_w, void *conv_state,
                    const float *g, const float *beta,
                    float *state, float *o,
                    float scale, float l2_eps,
                    int B, int Hk, int Hv, int dk, int dv, int dtype, int order, void *stream);

/*
 * gdn_gated_rmsnorm -- the gated RMSNorm at the output of the linear-attention layer
 * ("7.6 Qwen3.5: the linear-attention hybrid", section 7.6.2: o = RMSNorm(y) (.)
 * SiLU(z), z a separate projection of the layer input; the RMSNorm of section 7.6.3,
 * computed in fp32), over each (token, value head) row of dv outputs:
 *
 *   out[r][j] = y[r][j] / sqrt(mean_j y[r][j]^2 + eps) * gamma[j] * SiLU(z[r][j])
 *
 *   y      [rows][dv]  fp32, the recurrence output (o of the prefill or decode calls,
 *                      viewed as rows = tokens * Hv)
 *   z      [rows][dv]  element type `dtype`, the gate
 *   gamma  [dv]        element type `dtype`, the per-channel gain as applied (a
 *                      zero-centred RMSNorm weight w of section 7.6.3 is passed as 1 + w)
 *   out    [rows][dv]  element type `dtype`; may replace y (GDN_F32) or z exactly,
 *                      must not overlap gamma or partly overlap y or z
 * dv in {16, 32, 64, 128, 256}; eps >= 0 (the pages' RMSNorm uses 1e-6).
 * Errors: GDN_ERR_NULL_POINTER, GDN_ERR_BAD_SHAPE (rows < 0, bad eps),
 * GDN_ERR_UNSUPPORTED (dv, dtype), GDN_ERR_ALIAS, GDN_ERR_ALIGN.
 */
int gdn_gated_rmsnorm(const float *y, const void *z, const void *gamma, void *out,
                      long rows, int dv, float eps, int dtype, void *stream);

/*
 * gdn_decode_step_gated -- gdn_decode_step with the gated RMSNorm of
 * gdn_gated_rmsnorm applied to each head's output inside the same kernel: instead of
 * o, it writes out [B][Hv][dv] = RMSNorm(o) (.) gamma (.) SiLU(z) in element type
 * `dtype`, for z [B][Hv][dv] and gamma [dv] in that type and norm_eps >= 0.  Every
 * other argument is that of gdn_decode_step; out must not overlap any other argument.
 */
int gdn_decode_step_gated(const void *x, const void *conv_w, void *conv_state,
                          const float *g, const float *beta, float *state,
                          const void *z, const void *gamma, void *out,
                          float scale, float l2_eps, float norm_eps,
                          int B, int Hk, int Hv, int dk, int dv, int dtype, int order, void *stream);

/*
 * Linear-attention layer forward around the core ("7.6 Qwen3.5: the linear-attention
 * hybrid", section 7.6.2, layer widths of the section 7.6.1 table; cache handling of
 * "Hugging Face Transformers: Qwen3.5-MoE series explained", section 8.2): a bias-free
 * input projection of the layer input gives the pre-conv q|k|v, the output gate z and
 * two gate pre-activations a, b per value head; the conv + SiLU + L2 and the gated delta
 * rule follow; the output passes the gated RMSNorm with SiLU(z) and a bias-free output
 * projection.  The pages leave the gate maps open: here g = -softplus(a) (so the decay
 * exp(g) lies in (0, 1)) and beta = sigmoid(b).  Weights and the layer input are bf16;
 * products accumulate in fp32 on MFMA.  Weights are stored as a linear layer stores
 * them: W[out][in], y = x W^T.
 * Inside the layer calls the pre-conv q|k|v that the recurrence reads stays fp32, and so
 * do the layer's conv caches (the recurrent state amplifies a one-ulp bf16 change of its
 * inputs beyond the 2e-2 accuracy the layer is held to); z and the normalised output
 * that enters the output projection are bf16 (one bf16 rounding of a multiplicative gate
 * costs at most 2^-9 of the value).
 *
 * gdn_linear -- y = a w^T.
 *   a [M][K] bf16, w [N][K] bf16, y [M][N] bf16 (fp32 sums rounded to nearest even).
 *   K a positive multiple of 64, at most 2^20, and N a positive multiple of 4
 *   (GDN_ERR_UNSUPPORTED otherwise), M >= 0; y must not overlap a or w.
 */
int gdn_linear(const void *a, const void *w, void *y, int M, int N, int K, void *stream);

/*
 * gdn_in_proj -- the layer's input projection with its epilogue.
 *   hidden [T][E] bf16; w_in [conv_dim + Hv*dv + 2*Hv][E] bf16, rows in the order
 *   q|k|v (conv_dim), z (Hv*dv), a (Hv), b (Hv);
 *   x [T][conv_dim] bf16, z [T][Hv*dv] bf16: those columns of hidden w_in^T;
 *   g, beta [T][Hv] fp32: -softplus and sigmoid of the a and b columns.
 * E a positive multiple of 64 (at most 2^20), Hv*dv a multiple of 64, Hv <= 32, dk and dv
 * multiples of 16 (GDN_ERR_UNSUPPORTED otherwise).  Outputs must not overlap each other or
 * an input.
 */
int gdn_in_proj(const void *hidden, const void *w_in, void *x, void *z, float *g, float *beta,
                int T, int E, int Hk, int Hv, int dk, int dv, void *stream);

/*
 * gdn_layer_prefill -- the whole layer over packed sequences in one call: the input
 * projection (as gdn_in_proj, but x leaves it in fp32 and z in fp16, clamped to the fp16
 * range), gdn_prefill on the fp32 x, the gated RMSNorm of gdn_gated_rmsnorm over each
 * (token, value head) row (fp16 z, bf16 gamma and output), and gdn_linear with w_out.  Where the prefill runs its concurrent
 * schedule at dk = dv = 128 (one launch; at most a quarter of the compute units for the
 * state pass), the state pass forms the norm itself and the core output never reaches
 * memory; the row's mean square is then summed in another order than
 * gdn_gated_rmsnorm's, so a normalised value can differ from the separate pass's by one
 * bf16 ulp.  The environment variable GDN_LAYER_NORM_SEPARATE (set, not "0"; read at
 * every call) selects the separate pass everywhere.
 *   hidden [T][E], w_in as in gdn_in_proj, conv_w [conv_dim][4], gamma [dv] (the gain
 *   as applied), w_out [E][Hv*dv]: bf16.
 *   cu_seqlens, N, conv_state_in / conv_state_out [N][3][conv_dim] fp32,
 *   initial_state / final_state [N][Hv][dk][dv] fp32, scale, l2_eps, order: as in
 *   gdn_prefill (the same exact aliases allowed).
 *   out [T][E] bf16; norm_eps >= 0 the RMSNorm epsilon.
 *   workspace  at least gdn_layer_prefill_workspace_size(T, N, Hk, Hv, dk, dv) bytes
 *              (the prefill's workspace first, with its status word and wait bound,
 *              then x, z, y, g, beta, o and the norm's row-sum words); must not overlap any
 *              other argument.
 * dk = dv in {64, 128}; E and Hv as in gdn_in_proj.  out must not overlap an input.
 * The four steps run in order on `stream` (the prefill as in gdn_prefill).
 */
size_t gdn_layer_prefill_workspace_size(int T, int N, int Hk, int Hv, int dk, int dv);
int gdn_layer_prefill(const void *hidden, const void *w_in, const void *conv_w, const void *gamma,
                      const void *w_out, const int32_t *cu_seqlens, int N,
                      const void *conv_state_in, void *conv_state_out,
                      const float *initial_state, float *final_state, void *out,
                      float scale, float l2_eps, float norm_eps,
                      int T, int E, int Hk, int Hv, int dk, int dv, int order,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_layer_decode -- one token for each of B sequences through the layer: the input
 * projection of gdn_layer_prefill (x fp32), the decode step with the gated RMSNorm fused
 * (gdn_decode_step_gated, caches in place), gdn_linear with w_out.
 *   hidden [B][E] bf16; weights as in gdn_layer_prefill; conv_state [B][3][conv_dim]
 *   fp32 and state [B][Hv][dk][dv] fp32 in/out; out [B][E] bf16.
 *   workspace  at least gdn_layer_decode_workspace_size(B, E, Hk, Hv, dk, dv) bytes (x, z, g,
 *              beta, the normalised output and fp32 partial sums of the output projection,
 *              whose k extent is split over more compute units when B is small).
 * dk, dv in {16, 32, 64, 128}; E and Hv as in gdn_in_proj.
 */
size_t gdn_layer_decode_workspace_size(int B, int E, int Hk, int Hv, int dk, int dv);
int gdn_layer_decode(const void *hidden, const void *w_in, const void *conv_w, const void *gamma,
                     const void *w_out, void *conv_state, float *state, void *out,
                     float scale, float l2_eps, float norm_eps,
                     int B, int E, int Hk, int Hv, int dk, int dv, int order,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_layer_decode_noalloc -- for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops that forbid allocation): gdn_layer_decode with its
 * intermediate tensors in a scratch array that the library holds on each GPU it is loaded
 * on (64 MiB, kept until the process ends) instead of a caller's workspace.  Arguments and
 * results are those of gdn_layer_decode without the workspace.  Sizes whose intermediates
 * exceed the scratch (gdn_layer_decode_workspace_size(B, E, Hk, Hv, dk, dv) > 64 MiB, about
 * 680 rows at hidden 1024 and 16 value heads of 128) return GDN_ERR_WORKSPACE before
 * anything runs.  All calls on one GPU share its scratch: calls that overlap in time on one
 * GPU (two streams, or two threads) race; calls ordered on one stream do not.  No device
 * memory is allocated or freed by this call.
 */
int gdn_layer_decode_noalloc(const void *hidden, const void *w_in, const void *conv_w, const void *gamma,
                             const void *w_out, void *conv_state, float *state, void *out,
                             float scale, float l2_eps, float norm_eps,
                             int B, int E, int Hk, int Hv, int dk, int dv, int order, void *stream);

/* Static, human-readable name of a status code. */
const char *gdn_status_string(int status);

/* GDN_ABI_VERSION of the built library. */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */

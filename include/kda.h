/*
 * kda.h -- C ABI of the Kimi Delta Attention (KDA) layer core for AMD MI355X (gfx950).
 *
 * What the library computes (one head of one sequence; every (b, h) pair is
 * independent):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 *
 * with S in R^{dk x dv} (rows are key channels), g_t in R^dk the per-channel
 * log-decay and beta_t a scalar write strength.  Sources:
 *   - "Kimi K3 from Moonshot AI: 2.8 Trillion Parameters Unveiled", section
 *     "Kimi Delta Attention (KDA)": delta rule on the generalized Householder
 *     transformation; chunkwise ("piecewise parallel") reformulation.
 *   - "Kimi K3 Architecture Explained: KDA, Attention Residuals and LatentMoE",
 *     section "Token mixing: what KDA is and why 3:1": fixed-size recurrent
 *     state, error-correcting write, per-channel forget gate, output gate after
 *     a head-wise RMSNorm, constant per-token decode cost.
 *   - "Kimi K3: Engineering a 2.8 Trillion Parameter Frontier", section
 *     "Dimension 1: Sequence Length via Hybrid KDA-Gated MLA": log-decay
 *     bounded below by -5 through a scaled sigmoid, 16-token tiles whose
 *     cumulative log-decay stays in (-80, 0), dense matrix products on every
 *     causal tile.
 *
 * Conventions for every entry point:
 *   - All tensor arguments are DEVICE pointers owned by the caller, contiguous,
 *     row-major, in the layouts given per argument.  The library never
 *     allocates, frees or keeps a pointer after the call returns; scratch
 *     memory, where a call needs it, is a caller-provided workspace.
 *   - q, k, v, o, gate (and x, y) are in the io dtype (kda_dtype); g, beta,
 *     states and norm weights are always float32.
 *   - Every call is asynchronous on `stream` (NULL = the default stream).
 *     Arguments are validated on the host first; a non-OK status is returned
 *     BEFORE anything is launched, and no output is touched.  KDA_ERR_LAUNCH
 *     means the runtime refused the launch.  Faults inside a kernel surface at
 *     the caller's next synchronisation.
 *   - The library keeps no state between calls, never prints, and is safe to
 *     call from several host threads.
 *   - Supported head sizes: dk, dv in {16, 32, 64, 128}; any other value gives
 *     KDA_ERR_UNSUPPORTED_DIM.  Sizes B, T, H must be >= 1 (T >= 1); element
 *     offsets are 64-bit, so tensors above 2^31 elements are fine.
 *   - Precondition (documented; checked only in the input-check mode below):
 *     -5 <= g <= 0, as produced by g = -5 * sigmoid(.).  The chunked prefill
 *     relies on a 16-token sum of g staying above -80 so that exp(-sum) stays
 *     finite in float32/bfloat16.  Keys are expected to have unit L2 norm
 *     (the delta rule's write is a projection only then).
 *   - Magnitudes: values, initial states and outputs may take any finite
 *     float32 / bfloat16 magnitude.  The matrix-core prefill rounds the state,
 *     the values and the delta to float16 for its products; it keeps them in
 *     float16's normal range with an exact power-of-two scale per wavefront
 *     (the method is linear in (v, s0)), so no magnitude limit follows from
 *     that.  With the gated epilogue the row's mean square must stay finite in
 *     float32 (|o| below about 1e18).  The entry points that normalise raw q and
 *     k (the _prologue variants) form some matrix-core operands from the raw
 *     rows: there raw q and k norms between 2^-4 and 2^7 per token and head
 *     are supported (outside that range the float16 operands lose precision or
 *     overflow); all-zero rows are exact.
 *   - Input-check mode: with the environment variable KDA_CHECK_INPUTS=1 set
 *     when a call is made, kda_chunk_fwd*, kda_decode_step* and
 *     kda_decode_multi* first run a check kernel over their inputs and wait
 *     for it; if any floating-point input is not finite, any g is outside
 *     [-5, 0], or (prologue variants on the matrix-core path) a raw q or k norm
 *     lies outside [2^-4, 2^7] and is not zero, the call returns
 *     KDA_ERR_INPUT_RANGE and launches nothing else.  The check synchronises
 *     the stream (a debugging aid, not for graph capture).
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL_POINTER = 1,      /* a required pointer is NULL                         */
  KDA_ERR_BAD_SHAPE = 2,         /* B, T, H or rows < 1, or a size product overflows   */
  KDA_ERR_UNSUPPORTED_DIM = 3,   /* dk or dv not in {16, 32, 64, 128}                  */
  KDA_ERR_BAD_DTYPE = 4,         /* io dtype not a kda_dtype value                     */
  KDA_ERR_MISALIGNED = 5,        /* a pointer lacks the alignment its argument requires */
  KDA_ERR_ALIAS = 6,             /* an output overlaps an input it may not overlap     */
  KDA_ERR_BAD_ARGUMENT = 7,      /* a scalar argument is not finite or out of range    */
  KDA_ERR_LAUNCH = 8,            /* the HIP runtime rejected a kernel launch           */
  KDA_ERR_WORKSPACE = 9,         /* workspace NULL, too small or not 256-byte aligned  */
  KDA_ERR_INPUT_RANGE = 10       /* input-check mode: an input is not finite or out of
                                    its documented range (see KDA_CHECK_INPUTS)        */
} kda_status;

typedef enum {
  KDA_F32 = 0,   /* float32 q, k, v, o, gate: float32 arithmetic throughout            */
  KDA_BF16 = 1   /* bfloat16 q, k, v, o, gate: float32 accumulation, fp32 state        */
} kda_dtype;

/*
 * kda_chunk_fwd -- prefill: run the recurrence over T tokens for B x H heads.
 *
 * Computed chunkwise in 16-token tiles ("Kimi K3: Engineering ...", section
 * "Dimension 1"); the result equals the token-by-token recurrence up to
 * floating-point rounding.  With bfloat16 io and dk = dv = 128 it runs on the
 * matrix cores, one launch per segment of pairs of tiles: its first
 * workgroups walk the pairs of the segment of each head in order with the
 * running state on chip, while the other workgroups compute the
 * state-independent part of every pair of the next segment (the per-pair
 * records) into the workspace.
 * The state is written to memory only at segment boundaries (to s_out, or to
 * the workspace when s_out is NULL) and at the end.
 *
 *   q     [B, T, H, dk]  io dtype   queries
 *   k     [B, T, H, dk]  io dtype   keys (the method expects unit L2 norm; not checked)
 *   v     [B, T, H, dv]  io dtype   values
 *   g     [B, T, H, dk]  float32    log-decay, alpha = exp(g)
 *   beta  [B, T, H]      float32    write strength
 *   s0    [B, H, dk, dv] float32    initial state, or NULL for a zero state
 *   o     [B, T, H, dv]  io dtype   output, or NULL to compute the final state only.
 *                                   With gate != NULL, o receives the epilogue
 *                                   result y (see kda_gate_rmsnorm) instead of raw o.
 *   s_out [B, H, dk, dv] float32    final state, or NULL.  May equal s0 (in place);
 *                                   any other overlap with an input is KDA_ERR_ALIAS.
 *   gate  [B, T, H, dv]  io dtype   output-gate logits, or NULL for no epilogue
 *   norm_w [dv]          float32    RMSNorm weight, or NULL for a unit weight
 *   eps                             RMSNorm epsilon (> = 0, finite)
 *   scale                           output scale (finite)
 *   o and s_out may not both be NULL.  o may not overlap any input.
 *   workspace                       device scratch of at least workspace_bytes >=
 *                                   kda_chunk_fwd_workspace_size(B, T, H, dk, dv, io)
 *                                   bytes, 256-byte aligned, overlapping no other
 *                                   argument; its contents are undefined after the
 *                                   call.  May be NULL when that size is 0.
 *   Alignment: q, k, v, g, o and gate 16 bytes; beta, s0, s_out and norm_w 4 bytes.
 *   Calls that share a workspace must not run concurrently.
 */
kda_status kda_chunk_fwd(const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const float* s0,
                         void* o, float* s_out,
                         const void* gate, const float* norm_w, float eps,
                         int64_t B, int64_t T, int64_t H, int dk, int dv,
                         float scale, kda_dtype io, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * kda_chunk_fwd_workspace_size -- bytes of workspace kda_chunk_fwd needs for
 * these sizes: 0 for the vector-ALU path, otherwise two buffers of per-pair
 * records, each holding one segment of pairs of 16-token tiles of every head
 * (28,160 bytes per pair and head; about 96 MiB, at most 256 MiB unless one
 * pair of every head exceeds that), plus one float32 state per head.
 * Returns 0 for arguments kda_chunk_fwd would reject.
 */
size_t kda_chunk_fwd_workspace_size(int64_t B, int64_t T, int64_t H, int dk, int dv,
                                    kda_dtype io);

/*
 * kda_chunk_fwd_noalloc -- kda_chunk_fwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Every argument as in kda_chunk_fwd, without the
 * workspace: the call uses a fixed scratch array that the library declares in
 * device memory (kda_chunk_fwd_noalloc_scratch_bytes() = 64 MiB per GPU, held
 * until the process ends) and calls no allocator.  On the matrix-core path the
 * segments of per-pair records are shortened to fit it (more launches, so
 * slower than kda_chunk_fwd with its default workspace); results agree with
 * kda_chunk_fwd to rounding.  KDA_ERR_WORKSPACE when the scratch cannot hold
 * one pair of records per head of a launch group and the carried state (at
 * dk = dv = 128: H above about 540).  All calls on one GPU share its scratch:
 * calls that overlap in time on one GPU race, and the caller must serialise
 * them.
 */
kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                 const float* g, const float* beta, const float* s0,
                                 void* o, float* s_out, const void* gate, const float* norm_w,
                                 float eps, int64_t B, int64_t T, int64_t H, int dk, int dv,
                                 float scale, kda_dtype io, void* stream);

/* Bytes of the fixed scratch kda_chunk_fwd_noalloc uses on each GPU. */
size_t kda_chunk_fwd_noalloc_scratch_bytes(void);

/*
 * kda_chunk_fwd_prologue -- kda_chunk_fwd from the raw projections: q and k
 * are L2-normalised per head, and the decay and the write strength are formed
 * from their logits, all inside the kernels.
 *
 * "Kimi K3: Engineering a 2.8 Trillion Parameter Frontier", section
 * "Dimension 1": the log-decay is bounded below by a scaled sigmoid,
 * g = -5 sigmoid(a), so every retention factor exceeds e^-5; the write strength
 * is beta = sigmoid(b); "Kimi K3 Architecture Explained ...", section "Token
 * mixing": the delta-rule write replaces what the state predicts for a unit
 * key, so q <- q / max(|q|, 1e-12) and k likewise, per token and head.  Reading
 * a in the io dtype instead of float32 g halves the largest input (bfloat16:
 * 2 dk instead of 4 dk bytes per token and head), and no separate pass over
 * q, k, g or beta is needed.
 *
 *   q, k [B, T, H, dk]  io dtype   raw (unnormalised) queries and keys
 *   a    [B, T, H, dk]  io dtype   log-decay logits (in place of g)
 *   b    [B, T, H]      float32    write-strength logits (in place of beta)
 * Every other argument, alignment (a: 16 bytes) and aliasing rule as in
 * kda_chunk_fwd, including its workspace.
 */
kda_status kda_chunk_fwd_prologue(const void* q, const void* k, const void* v, const void* a,
                                  const float* b, const float* s0, void* o, float* s_out,
                                  const void* gate, const float* norm_w, float eps, int64_t B,
                                  int64_t T, int64_t H, int dk, int dv, float scale,
                                  kda_dtype io, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * kda_chunk_fwd_checkpoints -- kda_chunk_fwd that also keeps the state at
 * regular points of the sequence, for prefix caching (a fixed-size state per
 * cached prefix instead of a cache that grows with it; "Kimi K3 Architecture
 * Explained ...", section "Token mixing", and the prefix-caching remark of
 * "Kimi K3: Engineering a 2.8 Trillion Parameter Frontier").
 *
 * Every argument of kda_chunk_fwd, with the same meaning, plus
 *   ckpt       [B, T / ckpt_every, H, dk, dv] float32: entry [b, i, h] receives the
 *              state of (b, h) after its first (i + 1) * ckpt_every tokens (the
 *              state that kda_chunk_fwd over those tokens would leave in s_out).
 *              Must not overlap any other argument; 4-byte aligned.  With
 *              T < ckpt_every nothing is written.
 *   ckpt_every tokens between checkpoints, a positive multiple of 32 (two 16-token
 *              tiles), else KDA_ERR_BAD_SHAPE.
 * A checkpoint costs one store of the state per head (64 KiB at dk = dv = 128).
 */
kda_status kda_chunk_fwd_checkpoints(const void* q, const void* k, const void* v,
                                     const float* g, const float* beta, const float* s0,
                                     void* o, float* s_out, const void* gate,
                                     const float* norm_w, float eps, int64_t B, int64_t T,
                                     int64_t H, int dk, int dv, float scale, kda_dtype io,
                                     void* workspace, size_t workspace_bytes, float* ckpt,
                                     int64_t ckpt_every, void* stream);

/*
 * kda_chunk_fwd_varlen -- kda_chunk_fwd over N sequences of different lengths
 * packed along the token axis (a serving batch), with optional checkpoints.
 *
 * Sequence b occupies token rows cu_seqlens[b] .. cu_seqlens[b + 1] - 1 of the
 * packed tensors and runs its own recurrence from s0[b] (or zero) to s_out[b].
 * The work is laid out as for N sequences of max_len tokens: tokens past a
 * sequence's end are identity tokens (g = 0, beta = 0, k = 0), which leave the
 * state unchanged, and produce no output.
 *
 *   q, k, g    [total, H, dk]  (io dtype; g float32)      packed
 *   v, o, gate [total, H, dv]  io dtype                    packed (o, gate may be NULL as in
 *                                                          kda_chunk_fwd)
 *   beta       [total, H]      float32
 *   cu_seqlens [N + 1] int32 device array: 0 = cu[0] <= cu[1] <= ... <= cu[N] = total,
 *              every cu[b + 1] - cu[b] <= max_len.  Not checked; a violation gives
 *              undefined results (but no access outside the tensors: bounds are clamped
 *              into [0, total] and lengths to max_len).
 *   N, total, max_len  >= 1 (host values)
 *   s0, s_out  [N, H, dk, dv] float32, as in kda_chunk_fwd
 *   ckpt       [N, max_len / ckpt_every, H, dk, dv] float32 or NULL: entry [b, i, h] receives
 *              the state after the first (i + 1) * ckpt_every tokens of sequence b when it
 *              has that many (others are not written); ckpt_every as in
 *              kda_chunk_fwd_checkpoints (ignored when ckpt is NULL).
 *   workspace  at least kda_chunk_fwd_workspace_size(N, max_len, H, dk, dv, io) bytes.
 *   Every other argument, alignment and aliasing rule as in kda_chunk_fwd (cu_seqlens
 *   4 bytes, overlapping no output).
 */
kda_status kda_chunk_fwd_varlen(const void* q, const void* k, const void* v,
                                const float* g, const float* beta,
                                const int32_t* cu_seqlens, int64_t N, int64_t total,
                                int64_t max_len, const float* s0, void* o, float* s_out,
                                const void* gate, const float* norm_w, float eps, int64_t H,
                                int dk, int dv, float scale, kda_dtype io, void* workspace,
                                size_t workspace_bytes, float* ckpt, int64_t ckpt_every,
                                void* stream);

/*
 * kda_chunk_fwd_varlen_prologue -- kda_chunk_fwd_varlen from the raw
 * projections: q and k L2-normalised, g = -5 sigmoid(a) and beta = sigmoid(b)
 * formed in the kernels (as kda_chunk_fwd_prologue): a [total, H, dk] in the io
 * dtype in place of g, b [total, H] float32 in place of beta; everything else,
 * checkpoints included, as kda_chunk_fwd_varlen.
 */
kda_status kda_chunk_fwd_varlen_prologue(const void* q, const void* k, const void* v,
                                         const void* a, const float* b,
                                         const int32_t* cu_seqlens, int64_t N, int64_t total,
                                         int64_t max_len, const float* s0, void* o,
                                         float* s_out, const void* gate, const float* norm_w,
                                         float eps, int64_t H, int dk, int dv, float scale,
                                         kda_dtype io, void* workspace, size_t workspace_bytes,
                                         float* ckpt, int64_t ckpt_every, void* stream);

/*
 * kda_decode_step -- one token per sequence against a resident state.
 *
 * The constant-cost recurrent step ("Kimi K3 Architecture Explained ...",
 * section "Token mixing"): for every (b, h), with a = exp(g),
 *   p = (Diag(a) S)^T k,  u = beta (v - p),  S <- Diag(a) S + k u^T,  o = scale S^T q.
 * The state is read and written exactly once, in place.
 *
 *   q, k  [B, H, dk]     io dtype
 *   v     [B, H, dv]     io dtype
 *   g     [B, H, dk]     float32
 *   beta  [B, H]         float32
 *   state [B, H, dk, dv] float32    read and updated in place
 *   o     [B, H, dv]     io dtype   output (y when gate != NULL); must not be NULL
 *   gate  [B, H, dv]     io dtype   or NULL;  norm_w [dv] float32 or NULL;  eps, scale as above
 *   Alignment: state 16 bytes; every other pointer to its element size.
 */
kda_status kda_decode_step(const void* q, const void* k, const void* v,
                           const float* g, const float* beta, float* state,
                           void* o, const void* gate, const float* norm_w, float eps,
                           int64_t B, int64_t H, int dk, int dv,
                           float scale, kda_dtype io, void* stream);

/*
 * kda_decode_step_prologue -- kda_decode_step from the raw projections: q and
 * k L2-normalised, g = -5 sigmoid(a) and beta = sigmoid(b) formed in the kernel
 * (as kda_chunk_fwd_prologue): a [B, H, dk] in the io dtype in place of g,
 * b [B, H] float32 in place of beta; everything else as kda_decode_step.
 */
kda_status kda_decode_step_prologue(const void* q, const void* k, const void* v,
                                    const void* a, const float* b, float* state, void* o,
                                    const void* gate, const float* norm_w, float eps, int64_t B,
                                    int64_t H, int dk, int dv, float scale, kda_dtype io,
                                    void* stream);

/*
 * kda_decode_multi -- K consecutive tokens per sequence against the resident
 * state, with the state committed after a chosen number of them.
 *
 * The same recurrent step as kda_decode_step ("Kimi K3 Architecture Explained
 * ...", section "Token mixing"), applied to tokens t = 0 .. K-1 of every
 * (b, h) in order, the state held on chip between tokens.  Meant for
 * speculative decoding with draft tokens from the multi-token-prediction layer
 * ("Kimi K3: Engineering a 2.8 Trillion Parameter Frontier", section
 * "Infrastructure: The Physics of Running a 3T Model", EAGLE-3 item): a
 * call with n_commit all 0 verifies K draft tokens (outputs only; the state is
 * read once and not written), and a call with the accepted counts and o = NULL
 * advances the state by them.
 *
 *   q, k     [B, K, H, dk]  io dtype
 *   v        [B, K, H, dv]  io dtype
 *   g        [B, K, H, dk]  float32
 *   beta     [B, K, H]      float32
 *   state    [B, H, dk, dv] float32    read; overwritten in place by the state after the
 *                                      first n_commit[b] tokens of sequence b
 *   n_commit [B] int32 device array, or NULL for K.  A value is clamped into [0, K];
 *            0 leaves the state of every head of b untouched.
 *   o        [B, K, H, dv]  io dtype   outputs of all K tokens (y when gate != NULL), or NULL
 *                                      (then only the committed tokens are run)
 *   gate     [B, K, H, dv]  io dtype or NULL;  norm_w [dv] float32 or NULL;  eps, scale as above
 *   Alignment: state 16 bytes; every other pointer to its element size (n_commit 4).
 *   With K = 1 and n_commit NULL this computes what kda_decode_step does.
 */
kda_status kda_decode_multi(const void* q, const void* k, const void* v,
                            const float* g, const float* beta, float* state,
                            const int32_t* n_commit, void* o, const void* gate,
                            const float* norm_w, float eps, int64_t B, int64_t K, int64_t H,
                            int dk, int dv, float scale, kda_dtype io, void* stream);

/*
 * kda_decode_multi_prologue -- kda_decode_multi from the raw projections: q and
 * k L2-normalised, g = -5 sigmoid(a) and beta = sigmoid(b) formed in the kernel
 * (as kda_chunk_fwd_prologue): a [B, K, H, dk] in the io dtype in place of g,
 * b [B, K, H] float32 in place of beta; everything else as kda_decode_multi.
 */
kda_status kda_decode_multi_prologue(const void* q, const void* k, const void* v,
                                     const void* a, const float* b, float* state,
                                     const int32_t* n_commit, void* o, const void* gate,
                                     const float* norm_w, float eps, int64_t B, int64_t K,
                                     int64_t H, int dk, int dv, float scale, kda_dtype io,
                                     void* stream);

/*
 * kda_gate_rmsnorm -- the output epilogue on its own.
 *
 * "Kimi K3 Architecture Explained ...", section "Token mixing": the output
 * gate is applied after a head-wise RMSNorm.  For every row r (one head's dv
 * vector):  y[r] = x[r] / sqrt(mean(x[r]^2) + eps) * w * sigmoid(gate[r]).
 *
 *   x, gate, y [rows, dv]  io dtype  (y may equal x; any other overlap is KDA_ERR_ALIAS)
 *   norm_w     [dv]        float32, or NULL for a unit weight
 *   Alignment: every pointer 16 bytes.
 */
kda_status kda_gate_rmsnorm(const void* x, const void* gate, const float* norm_w, void* y,
                            int64_t rows, int dv, float eps, kda_dtype io, void* stream);

/*
 * kda_recurrent_bwd -- gradients of the token recurrence (the backward pass).
 *
 * The forward is the recurrence of kda_decode_step over T tokens ("Kimi K3
 * Architecture Explained ...", section "Token mixing"):
 *   S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T,  o_t = scale S_t^T q_t.
 * The pages give no backward pass; this returns the plain gradients of a loss
 * L given dL/do_t = dout[t] for every token and dL/dS_T = ds_final:
 *   dq, dk, dv, dg (with respect to the log-decay g), dbeta and ds0 (the initial state).
 * The state is recomputed from checkpoints every 64 tokens held in the workspace.
 *
 * Two kernels, chosen per call:
 *   bfloat16 io with q, k, v, dout, g, dq, dk, dv, dg all 16-byte aligned: the chunkwise
 *     pass on the matrix cores (16-token tiles; float16 operands with float32
 *     accumulation, the last tile's final-state terms as float16 value-and-rounding
 *     pairs).  Each gradient is within 2e-2 x its RMS of the float64 gradients (dq, dk,
 *     dv net of half a bfloat16 ulp), the forward's bfloat16-input bar.  Deterministic.
 *   otherwise (float32 io, or one of those tensors not 16-byte aligned, or the environment
 *     variable KDA_BWD_TOKEN=1): a token-serial float32 vector kernel, within 1e-4 x RMS.
 *
 *   q, k, v, dout     [B, T, H, 128]  io dtype
 *   g                 [B, T, H, 128]  float32;  beta [B, T, H] float32
 *   s0, ds_final      [B, H, 128, 128] float32 or NULL (zero initial state; no final-state term)
 *   dq, dk, dv        [B, T, H, 128]  io dtype, written
 *   dg                [B, T, H, 128]  float32, written;  dbeta [B, T, H] float32, written
 *   ds0               [B, H, 128, 128] float32 or NULL (not written)
 *   dk = dv = 128 only (else KDA_ERR_UNSUPPORTED_DIM).
 *   workspace         at least kda_recurrent_bwd_workspace_size(B, T, H, 128, 128) bytes, 16-byte
 *                     aligned; contents undefined after the call.
 *   Alignment: s0, ds_final, ds0 16 bytes; every other pointer to its element size.
 *   No output may overlap an input or another output.
 */
kda_status kda_recurrent_bwd(const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const float* s0, const void* dout,
                             const float* ds_final, void* dq, void* dk_out, void* dv_out,
                             float* dg, float* dbeta, float* ds0, int64_t B, int64_t T,
                             int64_t H, int dk, int dv, float scale, kda_dtype io,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_recurrent_bwd_ckpt -- kda_recurrent_bwd given the forward's states, for a
 * training step that runs the forward anyway: the chunkwise pass then skips its
 * own forward pass (one fifth to one sixth of its time at B=2, H=32, T=4096).
 *
 * Every argument of kda_recurrent_bwd, with the same meaning, plus
 *   ckpt   [B, T / 64, H, 128, 128] float32: entry [b, i, h] the state of (b, h) after
 *          its first 64 (i + 1) tokens, as kda_chunk_fwd_checkpoints with
 *          ckpt_every = 64 writes it over the same q, k, v, g, beta and s0 (not
 *          checked: other states give the gradients of another forward).  16-byte
 *          aligned; must not overlap an output.  Read only when T > 64.
 * bfloat16 io with q, k, v, dout, g, dq, dk, dv, dg 16-byte aligned only (the chunkwise
 * pass): else KDA_ERR_BAD_DTYPE or KDA_ERR_MISALIGNED.  The workspace is the one
 * kda_recurrent_bwd_workspace_size gives.  With the forward's own checkpoints the
 * gradients equal kda_recurrent_bwd's.
 */
kda_status kda_recurrent_bwd_ckpt(const void* q, const void* k, const void* v, const float* g,
                                  const float* beta, const float* s0, const void* dout,
                                  const float* ds_final, const float* ckpt, void* dq,
                                  void* dk_out, void* dv_out, float* dg, float* dbeta,
                                  float* ds0, int64_t B, int64_t T, int64_t H, int dk, int dv,
                                  float scale, kda_dtype io, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * kda_recurrent_bwd_workspace_size -- bytes of workspace kda_recurrent_bwd
 * needs: the larger of its two kernels' needs.  Token-serial: per (b, h), float32
 * states for ceil(T / 64) checkpoints plus 64 recomputed tokens (64 KiB each), then
 * four column-partial sums of dq, dk, dg and dbeta per token and head.  Chunkwise:
 * the forward's workspace, the state every 64 tokens and the adjoint at the end of
 * every 64 tokens (64 KiB each per head), and per 16-token tile a 24 KiB record,
 * 2 KiB of float32 16x16 factors and 26.5 KiB of products (about 5.3 KiB per token
 * and head in all; 2.0 GiB at B=2, H=32, T=4096).  0 for unsupported sizes.
 */
size_t kda_recurrent_bwd_workspace_size(int64_t B, int64_t T, int64_t H, int dk, int dv);

/*
 * kda_chunk_fwd_launches -- number of kernel launches one kda_chunk_fwd call
 * makes for these sizes (matrix-core path: one per segment of tiles plus one),
 * or 0 for arguments kda_chunk_fwd would reject.  For profiling and reporting.
 */
int64_t kda_chunk_fwd_launches(int64_t B, int64_t T, int64_t H, int dk, int dv, kda_dtype io);

/*
 * kda_chunk_fwd_kernel -- which prefill kernel kda_chunk_fwd launches for these
 * head sizes and io dtype: "kda_chunk_mfma" (bfloat16 matrix cores) or
 * "kda_chunk_valu" (float32 vector arithmetic), or NULL when the combination is
 * unsupported.  For profiling and reporting only; static storage.
 */
const char* kda_chunk_fwd_kernel(int dk, int dv, kda_dtype io);

/* Human-readable name of a status code (static storage; never NULL). */
const char* kda_status_string(kda_status s);

/* Library version, major * 10000 + minor * 100 + patch (0.2.0). */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */

/*
 * lin_attn.h -- C ABI of the gated delta-rule linear-attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation.  Per (batch b, head h) the library carries a fixed-size matrix
 * state and updates it token by token with a delta rule whose old content is
 * diluted by a data-dependent decay ("Evaluating Next-Gen Sparse MoE and
 * Long-Context LLMs", sec. 2, incremental linear attention; "Core Technologies
 * Behind Ultra-Long-Context Sparse MoE Large Models", sec. 2.1).  With the
 * state stored as h = S^T (d_k rows, d_v columns):
 *
 *     h_t = exp(g_t) * (h_{t-1} - beta_t k_t (k_t^T h_{t-1})) + beta_t k_t v_t^T
 *     o_t = h_t^T q_t
 *
 * The log-decay is bounded, g_t = -G * sigmoid(x_t) in [-G, 0] with G = 5 on
 * the pages ("Deep Dive: The Next Generation of Ultra-Long Context Sparse MoE
 * LLMs", sec. 3.3; "How Trillion-Scale Sparse MoE Models Achieve Million-Token
 * Long Context", sec. 3.2).  The forward pass is computed in 16-token tiles,
 * parallel inside a tile and recursive between tiles ("Deep Dive", sec. 3.2).
 *
 * Conventions for every entry point
 *  - Every array pointer is a DEVICE pointer owned by the caller.  The library
 *    never frees, keeps or reallocates caller memory, and allocates no device
 *    memory at run time; scratch space comes in as a caller-owned workspace
 *    (lin_attn_chunk_fwd_noalloc alone uses a buffer the library holds).
 *  - Arrays are dense, row-major, last dimension contiguous, and aligned to
 *    their element size; arrays the kernels access as vectors need more: q, k
 *    and v of lin_attn_chunk_fwd 16 bytes, its o 8 bytes in bf16, and S of
 *    lin_attn_decode_step 16 bytes.  Element type of q, k, v and o is given by `dtype`
 *    (LA_BF16 = bfloat16, LA_FP32 = float32); gate, beta, h0, hT and S are
 *    always float32.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns without waiting.  The return code reports host-side
 *    argument checks and launch errors only; device-side faults surface at the
 *    caller's next synchronisation.  No C++ exception crosses the ABI.
 *  - On any error nothing is enqueued and lin_attn_last_error() (thread-local)
 *    describes the reason.
 *  - Results are deterministic: the same inputs give bitwise-identical
 *    outputs on every call (no atomics in any reduction).
 *  - Calls may be made from several host threads; the library keeps no global
 *    mutable state besides the thread-local error text, a per-device cache
 *    of the compute-unit count (written once per device, read-only after) and
 *    the scratch buffer of lin_attn_chunk_fwd_noalloc.
 *  - Zero-size work (B, H or T equal to 0) is valid and enqueues nothing except
 *    that chunk_fwd with T = 0 copies h0 (or zeros) into hT.
 */
#ifndef LIN_ATTN_H
#define LIN_ATTN_H

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define LA_OK            0  /* success (work enqueued) */
#define LA_EINVAL        1  /* bad argument: NULL pointer, negative size,
                               misalignment, forbidden aliasing, bad enum */
#define LA_EUNSUPPORTED  2  /* valid but not built: head sizes outside the
                               supported set */
#define LA_ERANGE        3  /* a scalar parameter outside its allowed range,
                               or (lin_attn_check_inputs only) an input
                               value outside its range */
#define LA_EHIP          4  /* a HIP launch error; see lin_attn_last_error() */

/* Element types of q, k, v, o. */
#define LA_BF16 0
#define LA_FP32 1

/* Meaning of the `gate` array. */
#define LA_GATE_LOG            0  /* gate holds g_t itself; caller guarantees
                                     -G <= g_t <= 0 (checked only by
                                     lin_attn_check_inputs; the per-channel
                                     entry points clamp to [-G, 0])         */
#define LA_GATE_BOUNDED_LOGIT  1  /* gate holds x_t; g_t = -G * sigmoid(x_t) */

/*
 * lin_attn_chunk_fwd_workspace_size -- bytes of device workspace that
 * lin_attn_chunk_fwd needs for these sizes: 0 when it needs none (dtype
 * LA_FP32, or T = 0), and -1 (with lin_attn_last_error() set) when the sizes
 * are invalid or unsupported.  For LA_BF16 it is B * H * ceil(T / 32) * 6656:
 * the state-independent per-tile operators (the decay-weighted solve T diag(beta)
 * and the masked Q K^T block, see below) are computed once per head and kept
 * there between the two kernels of the pass.  When ceil(T / 32) >= 512 another
 * B * H * Dk * Dv * 4 bytes follow: long sequences may be processed in
 * stretches, and the fp32 state passes from one stretch to the next there.
 * When ceil(T / 32) >= 1536 a further B * H * (4 Dk Dv + 2 Dk^2) * 4 + 1024
 * bytes follow: with few heads a long sequence may run as three segments, the
 * middle one's state map formed beside the first (float32 states and maps,
 * and a zero block).
 */
long long lin_attn_chunk_fwd_workspace_size(int B, int T, int H, int Dk, int Dv, int dtype);

/*
 * lin_attn_chunk_fwd -- chunked forward pass over a whole sequence.
 *
 * Computes o_t for every token and the final state h_T of the recurrence
 * above, from the initial state h0, tile by tile (16 tokens per tile): inside
 * a tile the token interactions (the diagonal block) and the contribution of
 * the carried state (the "historical state -> current token" block) are
 * matrix products, and the state is carried from tile to tile ("Core
 * Technologies ...", sec. 2.1; "How Trillion-Scale ...", sec. 3.1).  In bf16
 * an intra-tile kernel first prepares every tile independently into the
 * workspace, then an inter-tile kernel carries the state.
 *
 *   q     [B, T, H, Dk]  dtype          queries
 *   k     [B, T, H, Dk]  dtype          keys (expected unit norm; not checked)
 *   v     [B, T, H, Dv]  dtype          values
 *   gate  [B, T, H]      float32        g_t or x_t, per gate_mode
 *   G     float, 0 <= G <= 16           decay bound (5 on the pages)
 *   beta  [B, T, H]      float32        write strengths, expected in [0, 1]
 *   h0    [B, H, Dk, Dv] float32 or NULL (NULL = zero initial state)
 *   o     [B, T, H, Dv]  dtype          output, rounded to nearest-even from
 *                                       float32 when dtype is LA_BF16
 *   hT    [B, H, Dk, Dv] float32 or NULL (NULL = final state not written)
 *   workspace, workspace_bytes
 *                        device scratch of at least
 *                        lin_attn_chunk_fwd_workspace_size(...) bytes, 256-byte
 *                        aligned, owned by the caller; its contents on entry do
 *                        not matter and are overwritten.  May be NULL when the
 *                        size is 0.  Two calls in flight at the same time must
 *                        not share a workspace.
 *   Dk in {64, 128}; Dv a multiple of 16 in [16, 256]; B, T, H >= 0.
 *
 * Aliasing: o must not overlap any input.  hT may be the very same pointer as
 * h0 (the state is then updated in place); any other overlap of hT with an
 * input or with o is rejected, and so is any overlap of the workspace with an
 * argument array.  T need not be a multiple of 16: the last tile
 * behaves as if padded with tokens q = k = v = 0, g = 0, beta = 0, which leave
 * the state unchanged.
 */
int lin_attn_chunk_fwd(const void* q, const void* k, const void* v,
                       const float* gate, int gate_mode, float G,
                       const float* beta, const float* h0,
                       void* o, float* hT,
                       int B, int T, int H, int Dk, int Dv, int dtype,
                       void* workspace, long long workspace_bytes,
                       void* stream);

/*
 * lin_attn_chunk_fwd_noalloc -- lin_attn_chunk_fwd for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same computation, arguments, rules
 * and errors, without the workspace arguments.  The scratch comes from a
 * buffer the library owns, 64 MiB per GPU (held from the library's load on
 * that GPU until the process ends); sizes whose workspace
 * (lin_attn_chunk_fwd_workspace_size) exceeds 64 MiB are rejected with
 * LA_EINVAL.  Allocates nothing (no hipMalloc, hipFree or allocating library
 * call).  Every call on one GPU shares that GPU's buffer and the buffer keeps
 * the last call's contents (nothing in it needs to start at zero): calls that
 * may overlap in time on the same GPU race, so serialise them, e.g. on one
 * stream.
 */
int lin_attn_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                               const float* gate, int gate_mode, float G,
                               const float* beta, const float* h0,
                               void* o, float* hT,
                               int B, int T, int H, int Dk, int Dv, int dtype,
                               void* stream);

/*
 * lin_attn_chunk_fwd_raw -- lin_attn_chunk_fwd with the input preparation
 * fused into its intra-tile kernel: q and k are given as they come from their
 * projections and are L2-normalised per (token, head) inside the pass, in
 * fp32 from the given values (a zero vector stays zero), and beta_logit holds
 * x_beta with beta = sigmoid(x_beta).  The gate is given as for
 * lin_attn_chunk_fwd (gate_mode).  Same arguments, layouts, workspace, rules
 * and errors otherwise; dtype LA_BF16 or LA_FP32.  For LA_BF16 the
 * normalisation is folded into the per-tile operators (1/|k_t| and 1/|q_t|
 * scale rows and columns of the in-tile products and the decay factors); for
 * LA_FP32 the fused kernel scales the rows as it loads them.  Either way q
 * and k are read as given and never rewritten.
 */
int lin_attn_chunk_fwd_raw(const void* q, const void* k, const void* v,
                           const float* gate, int gate_mode, float G,
                           const float* beta_logit, const float* h0,
                           void* o, float* hT,
                           int B, int T, int H, int Dk, int Dv, int dtype,
                           void* workspace, long long workspace_bytes,
                           void* stream);

/*
 * lin_attn_chunk_fwd_raw_affine -- lin_attn_chunk_fwd_raw with the gate's
 * per-head affine pre-activation fused in: gate_x holds x_t [B, T, H] float32
 * and
 *
 *     g_t = -G * sigmoid(a_h * x_t + b_h)
 *
 * with a = gate_scale[h], b = gate_bias[h] (device arrays of H float32, 4-byte
 * aligned; NULL stands for a = 1, resp. b = 0, and both NULL is
 * lin_attn_chunk_fwd_raw in LA_GATE_BOUNDED_LOGIT mode).  The pages write the
 * bounded decay as a sigmoid of an affine function of the layer's input,
 * scaled by the bound ("Evaluating Next-Gen ...", sec. 2 item 3; "Core
 * Technologies ...", sec. 2.2); a and b scale and shift the logit of each
 * head, so that a caller holding x needs no separate pass over it.  The
 * affine map and the sigmoid are evaluated in float32 inside the intra-tile
 * kernel.  Arguments, layouts, workspace (lin_attn_chunk_fwd_workspace_size),
 * rules and errors as lin_attn_chunk_fwd_raw; LA_EINVAL also when gate_scale
 * or gate_bias is misaligned or overlaps o, hT or the workspace.  Non-finite
 * a or b give what the formula gives (a NaN logit gives a NaN decay).
 */
int lin_attn_chunk_fwd_raw_affine(const void* q, const void* k, const void* v,
                                  const float* gate_x, float G, const float* gate_scale,
                                  const float* gate_bias, const float* beta_logit,
                                  const float* h0, void* o, float* hT,
                                  int B, int T, int H, int Dk, int Dv, int dtype,
                                  void* workspace, long long workspace_bytes,
                                  void* stream);

/*
 * lin_attn_chunk_fwd_channel -- lin_attn_chunk_fwd with one log-decay per key
 * channel: gate is [B, T, H, Dk] float32 (16-byte aligned), g_t[c] in [-G, 0]
 * (LA_GATE_LOG) or g_t[c] = -G * sigmoid(x_t[c]) (LA_GATE_BOUNDED_LOGIT).
 *
 * The pages call the decay "per-token decay factors" and bound the log-decay
 * elementwise so that, inside a 16-token tile, the reciprocal of the
 * cumulative decay stays finite ("Core Technologies ...", sec. 2.1 and 2.3;
 * "How Trillion-Scale ...", sec. 3.1 and 3.2).  With a decay per channel that
 * reciprocal enters the tile products.  The recurrence (h = S^T):
 *
 *     d_t = diag(exp(g_t)) h_{t-1}
 *     h_t = d_t - beta_t k_t (k_t^T d_t) + beta_t k_t v_t^T,   o_t = h_t^T q_t
 *
 * i.e. the decay acts on the key side of the old state first, then the
 * delta-rule erase and write act on the decayed state; with every channel
 * equal it is lin_attn_chunk_fwd.  LA_FP32 computes in float32 throughout;
 * LA_BF16 forms the tile operators in float32 and runs the products with the
 * carried state on bf16 matrix cores (float32 state and accumulation).
 * Arguments, layouts, alignment, aliasing rules, tail handling and errors as
 * lin_attn_chunk_fwd, except: the workspace holds one record per tile and
 * head (lin_attn_chunk_fwd_channel_workspace_size bytes, for both dtypes), and
 * 0 <= G <= 10 (LA_ERANGE beyond: the tile operands reach exp(8 G)).
 */
int lin_attn_chunk_fwd_channel(const void* q, const void* k, const void* v,
                               const float* gate, int gate_mode, float G,
                               const float* beta, const float* h0, void* o, float* hT,
                               int B, int T, int H, int Dk, int Dv, int dtype,
                               void* workspace, long long workspace_bytes, void* stream);

/*
 * lin_attn_chunk_fwd_channel_workspace_size -- device workspace bytes of
 * lin_attn_chunk_fwd_channel: B * H * ceil(T / 16) * R, with R (Dk = 128 / 64)
 * = 27,136 / 14,592 for LA_FP32 (the state-independent operators of each
 * 16-token tile, prepared once per head); for LA_BF16 the larger of that with
 * R = 18,944 / 10,496 and B * H * ceil(T / 32) * R2 with R2 = 31,232 / 18,688
 * (the operators of each 32-token pair of tiles: the pass steps the state
 * over tiles or pairs of tiles, whichever fills the device better);
 * 0 when T = 0; -1 (with
 * lin_attn_last_error() set) for invalid or unsupported sizes.
 */
long long lin_attn_chunk_fwd_channel_workspace_size(int B, int T, int H, int Dk, int Dv,
                                                   int dtype);

/*
 * lin_attn_chunk_fwd_varlen_workspace_size -- bytes of device workspace that
 * lin_attn_chunk_fwd_varlen needs: H * (T / 32 + nseq + 1) * 6656 for LA_BF16
 * (one 6656-byte record slot per 32 tokens of each packed sequence, as in
 * lin_attn_chunk_fwd, plus one spare slot per sequence for its ragged end),
 * 0 for LA_FP32, -1 (with lin_attn_last_error() set) for invalid or
 * unsupported sizes.
 */
long long lin_attn_chunk_fwd_varlen_workspace_size(int T, int nseq, int H, int Dk, int Dv,
                                                   int dtype);

/*
 * lin_attn_chunk_fwd_varlen -- the same forward pass over packed sequences of
 * different lengths (chunked prefill of a serving batch, "Evaluating Next-Gen
 * ...", sec. 4): sequence s is tokens [cu_seqlens[s], cu_seqlens[s + 1]) of
 * one packed sequence of T tokens, starts from its own initial state h0[s]
 * and never sees another sequence's state.  Each sequence is processed
 * exactly as lin_attn_chunk_fwd processes a sequence of its length (its own
 * tiles start at its first token).
 *
 *   q, k        [T, H, Dk]  dtype        (a batch of one packed sequence)
 *   v, o        [T, H, Dv]  dtype
 *   gate, beta  [T, H]      float32
 *   h0, hT      [nseq, H, Dk, Dv] float32, or NULL as in lin_attn_chunk_fwd
 *   cu_seqlens  DEVICE array of nseq + 1 int32 offsets: 0 = cu[0] <= cu[1] <=
 *               ... <= cu[nseq] = T.  The values are read on the device only
 *               (no synchronisation); they are clamped to [0, T] so that any
 *               values stay memory-safe, but offsets that are not
 *               non-decreasing give undefined results.  Empty sequences are
 *               allowed (their hT is h0, or zeros).
 *   workspace   lin_attn_chunk_fwd_varlen_workspace_size(...) bytes, as in
 *               lin_attn_chunk_fwd (none, and may be NULL, for LA_FP32).
 *   dtype       LA_BF16 or LA_FP32 (the fp32 path: one fused kernel, one
 *               workgroup per sequence, head and 16 columns of d_v).
 *   Dk in {64, 128}; Dv a multiple of 16 in [16, 256]; T, nseq, H >= 0.
 * Alignment and aliasing rules are those of lin_attn_chunk_fwd.
 */
int lin_attn_chunk_fwd_varlen(const void* q, const void* k, const void* v,
                              const float* gate, int gate_mode, float G,
                              const float* beta, const float* h0,
                              void* o, float* hT, const int* cu_seqlens, int nseq,
                              int T, int H, int Dk, int Dv, int dtype,
                              void* workspace, long long workspace_bytes,
                              void* stream);

/*
 * lin_attn_chunk_fwd_varlen_raw -- lin_attn_chunk_fwd_varlen with the input
 * preparation of lin_attn_chunk_fwd_raw: q and k as given (L2-normalised per
 * token and head inside the pass), beta_logit holding x_beta.  Same arguments,
 * workspace, rules and errors otherwise (both dtypes).
 */
int lin_attn_chunk_fwd_varlen_raw(const void* q, const void* k, const void* v,
                                  const float* gate, int gate_mode, float G,
                                  const float* beta_logit, const float* h0,
                                  void* o, float* hT, const int* cu_seqlens, int nseq,
                                  int T, int H, int Dk, int Dv, int dtype,
                                  void* workspace, long long workspace_bytes,
                                  void* stream);

/*
 * lin_attn_chunk_fwd_varlen_raw_affine -- lin_attn_chunk_fwd_varlen_raw with
 * the gate of lin_attn_chunk_fwd_raw_affine: gate_x [T, H] holds x_t and
 * g_t = -G * sigmoid(gate_scale[h] * x_t + gate_bias[h]).  Arguments,
 * workspace, rules and errors as lin_attn_chunk_fwd_varlen_raw and
 * lin_attn_chunk_fwd_raw_affine.
 */
int lin_attn_chunk_fwd_varlen_raw_affine(const void* q, const void* k, const void* v,
                                         const float* gate_x, float G,
                                         const float* gate_scale, const float* gate_bias,
                                         const float* beta_logit, const float* h0,
                                         void* o, float* hT, const int* cu_seqlens, int nseq,
                                         int T, int H, int Dk, int Dv, int dtype,
                                         void* workspace, long long workspace_bytes,
                                         void* stream);

/*
 * lin_attn_decode_step -- one new token per (b, h), state updated in place.
 *
 * Constant-state recurrent inference: each sequence advances its d_k x d_v
 * state by one token and reads it out ("Evaluating Next-Gen ...", sec. 2
 * item 2 and sec. 4, constant-state linear attention layers in serving).
 * Equivalent to lin_attn_chunk_fwd with T = 1 and hT = h0 = S.
 *
 *   q, k  [B, H, Dk] dtype;  v [B, H, Dv] dtype
 *   gate, beta [B, H] float32 (gate per gate_mode, as above)
 *   S     [B, H, Dk, Dv] float32, read and overwritten in place
 *   o     [B, H, Dv] dtype, output (reads the updated state)
 *   Dk in {64, 128}; Dv in {64, 128}.
 * o must not overlap any input; S must not overlap q, k, v, gate, beta or o.
 */
int lin_attn_decode_step(const void* q, const void* k, const void* v,
                         const float* gate, int gate_mode, float G,
                         const float* beta, float* S, void* o,
                         int B, int H, int Dk, int Dv, int dtype,
                         void* stream);

/*
 * lin_attn_chunk_fwd_channel_varlen_workspace_size -- device workspace bytes of
 * lin_attn_chunk_fwd_channel_varlen: H * (T / 16 + nseq + 1) * R with R as in
 * lin_attn_chunk_fwd_channel_workspace_size (one record slot per 16 tokens of
 * each packed sequence plus one spare slot per sequence for its ragged end);
 * for LA_BF16 the larger of that and H * (T / 32 + nseq + 1) * R2 (slots of
 * 32-token pairs);
 * -1 (with lin_attn_last_error() set) for invalid or unsupported sizes.
 */
long long lin_attn_chunk_fwd_channel_varlen_workspace_size(int T, int nseq, int H, int Dk,
                                                           int Dv, int dtype);

/*
 * lin_attn_chunk_fwd_channel_varlen -- lin_attn_chunk_fwd_channel over packed
 * sequences of different lengths (chunked prefill of a serving batch,
 * "Evaluating Next-Gen ...", sec. 4): sequence s is tokens [cu_seqlens[s],
 * cu_seqlens[s + 1]) of one packed sequence of T tokens, starts from its own
 * h0[s] and is computed exactly as lin_attn_chunk_fwd_channel computes a
 * sequence of its length.  Arguments and rules as lin_attn_chunk_fwd_varlen
 * (q, k [T, H, Dk]; v, o [T, H, Dv]; beta [T, H]; h0, hT [nseq, H, Dk, Dv];
 * device offsets, clamped to [0, T], read only on the device; empty sequences
 * allowed), except: gate is [T, H, Dk] float32 (16-byte aligned); both dtypes
 * are supported; 0 <= G <= 10.
 */
int lin_attn_chunk_fwd_channel_varlen(const void* q, const void* k, const void* v,
                                      const float* gate, int gate_mode, float G,
                                      const float* beta, const float* h0, void* o, float* hT,
                                      const int* cu_seqlens, int nseq, int T, int H, int Dk,
                                      int Dv, int dtype, void* workspace,
                                      long long workspace_bytes, void* stream);

/*
 * lin_attn_decode_step_channel -- lin_attn_decode_step with one log-decay per
 * key channel: gate is [B, H, Dk] float32 (g or its logit, per gate_mode), and
 * the step is the per-channel recurrence of lin_attn_chunk_fwd_channel
 * (decay on the key side of the old state, then erase and write), so a
 * per-channel prefill hands its hT to this step unchanged.  Arguments, layouts,
 * in-place S, supported sizes and errors as lin_attn_decode_step, except
 * 0 <= G <= 10.
 */
int lin_attn_decode_step_channel(const void* q, const void* k, const void* v,
                                 const float* gate, int gate_mode, float G, const float* beta,
                                 float* S, void* o, int B, int H, int Dk, int Dv, int dtype,
                                 void* stream);

/*
 * lin_attn_chunk_bwd_workspace_size -- device workspace bytes lin_attn_chunk_bwd
 * needs.  Every 16-token tile and head takes a 3,200-byte record.  With
 * LA_BF16 and Dv <= 128, the state is kept at every second tile and the
 * gradient of the state at every fourth, as packed bf16 (hi, lo) words: B * H *
 * (ceil(T / 16) * 3200 + ceil(T / 64) * 12 * Dk * Dv) bytes.  Otherwise
 * (LA_FP32, or Dv > 128) both are kept at every tile in float32: B * H *
 * ceil(T / 16) * (3200 + 8 * Dk * Dv) bytes.  -1 on invalid sizes (message in
 * lin_attn_last_error).
 */
long long lin_attn_chunk_bwd_workspace_size(int B, int T, int H, int Dk, int Dv, int dtype);

/*
 * lin_attn_chunk_bwd -- reverse mode of lin_attn_chunk_fwd, for training.
 *
 * The pages frame the bounded decay around BF16 training ("Core Technologies
 * ...", sec. 2.3) and give the tiled forward pass ("Deep Dive ...", sec. 3.2);
 * they print no backward pass.  This entry point returns the gradients of
 * L = <o, dout> + <hT, dhT> with respect to every input of the forward pass,
 * computed over 16-token tiles with float32 accumulation and float32 carried
 * states (the forward states are recomputed, the state gradient is carried
 * backwards tile by tile).  LA_FP32 runs its products on the float32 matrix
 * cores.  LA_BF16 with Dv <= 128 runs them on the bf16 matrix cores, every
 * float32 operand split into bf16 hi + lo parts (relative error 2^-16 per
 * operand; the bf16 inputs enter exactly), and keeps the states only at
 * every second tile and the state gradients at every fourth, rebuilding
 * those between inside the gradient kernel.
 *
 *   q, k, v, gate, beta, h0, gate_mode, G, sizes, dtype: as lin_attn_chunk_fwd
 *     (q and k 16-byte aligned; h0 may be NULL = zeros)
 *   dout  [B, T, H, Dv] dtype: upstream gradient of o
 *   dhT   [B, H, Dk, Dv] float32 or NULL (zero): upstream gradient of hT
 *   dq, dk [B, T, H, Dk], dv [B, T, H, Dv] float32 outputs, 16-byte aligned
 *   dgate [B, T, H] float32 output: dL/dg (LA_GATE_LOG) or dL/dx
 *         (LA_GATE_BOUNDED_LOGIT, through g = -G * sigmoid(x))
 *   dbeta [B, T, H] float32 output
 *   dh0   [B, H, Dk, Dv] float32 output, or NULL (not written)
 *   workspace >= lin_attn_chunk_bwd_workspace_size(...) bytes, 256-byte
 *         aligned, caller-owned, clobbered.
 * No output may overlap an input, another output or the workspace (LA_EINVAL).
 * T = 0 writes dh0 = dhT (or zeros) and nothing else.  Deterministic: the
 * same inputs give bitwise-identical outputs.
 */
int lin_attn_chunk_bwd(const void* q, const void* k, const void* v,
                       const float* gate, int gate_mode, float G,
                       const float* beta, const float* h0,
                       const void* dout, const float* dhT,
                       float* dq, float* dk, float* dv,
                       float* dgate, float* dbeta, float* dh0,
                       int B, int T, int H, int Dk, int Dv, int dtype,
                       void* workspace, long long workspace_bytes, void* stream);

/*
 * lin_attn_chunk_bwd_segmented_workspace_size -- device workspace bytes of
 * lin_attn_chunk_bwd_segmented: what lin_attn_chunk_bwd needs for one
 * sequence of min(T, segment_tokens) tokens (rounded up to 256 bytes), plus
 * H * Dk * Dv * 4 bytes for each of the ceil(T / segment_tokens) + 1 carried
 * states (the states at segment starts and two state-gradient buffers),
 * whatever B.  -1 (message in lin_attn_last_error) on invalid sizes, for
 * anything but LA_BF16 with Dk 64 or 128 and Dv <= 128, or when
 * segment_tokens is not a positive multiple of 64.
 */
long long lin_attn_chunk_bwd_segmented_workspace_size(int B, int T, int H, int Dk, int Dv,
                                                      int dtype, int segment_tokens);

/*
 * lin_attn_chunk_bwd_segmented -- lin_attn_chunk_bwd with a workspace bounded
 * by the segment length instead of the sequence length (for long sequences:
 * at B=1 H=8 T=1048576 d=128 the one-pass workspace is 27.4 GB; with
 * segments of 65536 tokens it is 1.7 GB).  Each sequence is cut into segments
 * of segment_tokens tokens (a multiple of 64, so that every tile, group of
 * four tiles and stored state falls where it falls in one pass): a first pass
 * carries the forward state through the segments and keeps it only at
 * segment starts; a second pass takes the segments backwards, each one a
 * reverse pass from its start state with the gradient of its end state
 * carried from the segment after it.  The results are bitwise those of
 * lin_attn_chunk_bwd; the forward states are computed twice.
 *
 *   arguments: as lin_attn_chunk_bwd (dtype LA_BF16, Dk 64 or 128,
 *     Dv <= 128), plus segment_tokens
 *   workspace >= lin_attn_chunk_bwd_segmented_workspace_size(...) bytes,
 *     256-byte aligned, caller-owned, clobbered.
 * Errors: as lin_attn_chunk_bwd; LA_EINVAL for another dtype or shape, or a
 * segment length that is not a positive multiple of 64.
 */
int lin_attn_chunk_bwd_segmented(const void* q, const void* k, const void* v,
                                 const float* gate, int gate_mode, float G,
                                 const float* beta, const float* h0,
                                 const void* dout, const float* dhT,
                                 float* dq, float* dk, float* dv,
                                 float* dgate, float* dbeta, float* dh0,
                                 int B, int T, int H, int Dk, int Dv, int dtype,
                                 int segment_tokens, void* workspace,
                                 long long workspace_bytes, void* stream);

/*
 * lin_attn_chunk_bwd_varlen_workspace_size -- bytes of device workspace that
 * lin_attn_chunk_bwd_varlen needs: H * (T / 16 + nseq + 1) tile slots (one per
 * 16 tokens of each packed sequence plus one spare per sequence for its
 * ragged end), each holding what lin_attn_chunk_bwd keeps per tile (3200 +
 * 8 * Dk * Dv bytes; with LA_BF16 and Dv <= 128 only the 3200-byte record,
 * plus H * (T / 64 + nseq + 1) group slots of 12 * Dk * Dv bytes for the
 * states kept at every second and the state gradients at every fourth
 * tile); -1 (with lin_attn_last_error() set) for
 * invalid sizes.
 */
long long lin_attn_chunk_bwd_varlen_workspace_size(int T, int nseq, int H, int Dk, int Dv,
                                                   int dtype);

/*
 * lin_attn_chunk_bwd_varlen -- the reverse pass of lin_attn_chunk_fwd_varlen
 * (training on packed sequences): sequence s is tokens [cu_seqlens[s],
 * cu_seqlens[s + 1]) of one packed sequence of T tokens, with its own h0[s]
 * and dhT[s]; gradients never cross from one sequence to another.  Each
 * sequence gets exactly the gradients lin_attn_chunk_bwd gives a sequence of
 * its length.
 *
 *   q, k, dq, dk            [T, H, Dk]   (q, k dtype; dq, dk float32)
 *   v, dout, dv             [T, H, Dv]   (v, dout dtype; dv float32)
 *   gate, beta, dgate, dbeta [T, H]      float32
 *   h0, dhT, dh0            [nseq, H, Dk, Dv] float32, or NULL as in
 *                           lin_attn_chunk_bwd
 *   cu_seqlens  DEVICE array of nseq + 1 int32 offsets, as in
 *               lin_attn_chunk_fwd_varlen (read on the device only, clamped
 *               to [0, T]; empty sequences allowed: their dh0 is dhT).
 *   workspace   lin_attn_chunk_bwd_varlen_workspace_size(...) bytes,
 *               256-byte aligned, caller-owned, clobbered.
 * dtype LA_BF16 or LA_FP32; sizes, alignment, aliasing rules and errors as
 * lin_attn_chunk_bwd.  Deterministic.
 */
int lin_attn_chunk_bwd_varlen(const void* q, const void* k, const void* v,
                              const float* gate, int gate_mode, float G,
                              const float* beta, const float* h0,
                              const void* dout, const float* dhT,
                              float* dq, float* dk, float* dv,
                              float* dgate, float* dbeta, float* dh0,
                              const int* cu_seqlens, int nseq,
                              int T, int H, int Dk, int Dv, int dtype,
                              void* workspace, long long workspace_bytes, void* stream);

/*
 * lin_attn_gate -- the bounded log-decay on its own: g[i] = -G * sigmoid(x[i])
 * for i < n ("Deep Dive ...", sec. 3.3; "Core Technologies ...", sec. 2.2).
 * x and g are float32 device arrays of n elements (g may equal x for an
 * in-place transform; other overlaps are rejected).  0 <= G <= 16.
 */
int lin_attn_gate(const float* x, float G, float* g, long long n, void* stream);

/*
 * lin_attn_check_inputs -- opt-in debug range check of a forward pass's inputs
 * (the bounded log-decay lies in [-G, 0]: "Deep Dive: The Next Generation of
 * Ultra-Long Context Sparse MoE LLMs", sec. 3.3; beta is a write strength in
 * [0, 1]).  The hot entry points never read their inputs on the host and do
 * not check values; a caller that wants the check calls this first.
 *
 *   q, k   [ntok, H, Dk] dtype;  v [ntok, H, Dv] dtype
 *   gate   [ntok, H] float32, or [ntok, H, Dk] when channel != 0
 *   beta   [ntok, H] float32;  h0 [nstate, H, Dk, Dv] float32 or NULL
 *   ntok   tokens (B * T for a batch, T for packed sequences); nstate the
 *          number of initial states (B, or nseq)
 *   flags  DEVICE pointer to one caller-owned unsigned int (scratch; cleared
 *          and written by the check)
 * Returns LA_ERANGE when any q, k, v or h0 element is not finite, any beta is
 * outside [0, 1] (or NaN), or any gate value is outside [-G, 0] or not finite
 * (LA_GATE_LOG) or NaN (LA_GATE_BOUNDED_LOGIT: +-inf logits are in range, they
 * give g = 0 and g = -G); the message names every class found.  LA_OK when
 * everything is in range.  Unlike every other entry point this one BLOCKS: it
 * enqueues two small kernels on `stream`, then synchronises the stream and
 * copies the flag to the host.  Sizes and dtype as lin_attn_chunk_fwd
 * (alignment: 4 bytes).
 */
int lin_attn_check_inputs(const void* q, const void* k, const void* v, const float* gate,
                          int gate_mode, float G, const float* beta, const float* h0,
                          long long ntok, int nstate, int H, int Dk, int Dv, int channel,
                          int dtype, unsigned* flags, void* stream);

/* Text of the last error on the calling thread ("" if none). */
const char* lin_attn_last_error(void);

/* Library ABI version (major * 100 + minor). */
int lin_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIN_ATTN_H */

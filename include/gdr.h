/*
 * gdr.h -- C ABI of libgdr, the gated delta-rule recurrence on AMD Instinct
 * MI355X (gfx950).
 *
 * The operation (page "How the New Flash Models Work: Inside GLM-5.3-Flash and
 * Qwen3.8-Flash-Next", section "Linear attention: a fixed-size memory in place
 * of the cache"): per head, a d_v x d_k state S is carried over the tokens of a
 * sequence and updated once per token,
 *
 *     S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = scale * S_t q_t,
 *
 * where alpha_t = exp(log_alpha_t) is one value per (token, head) for Gated
 * DeltaNet (the section's first equation, decay "per head") and one value per
 * key channel for Kimi Delta Attention (the section's second equation; page
 * "GLM-5.3-Flash vs Qwen3.8-Flash-Next: Two Labs, One Architecture", section
 * "The four shared design choices": KDA gates per channel, GDN per head).
 * The state is held in FP32 (same first section: recurrent state is often
 * held in FP32).  The pages print no query scale; `scale` multiplies the
 * readout only and is 1 for the equations as printed.
 *
 * Two phases, as the pages' serving discussion separates them (page "How the
 * New Flash Models Work...", section "Serving: prefill and decode are
 * different problems"): a chunked prefill over whole prompts, and a decode
 * step of one token per sequence that reads and writes the state in place.
 * The prefill's final state has exactly the layout the decode step takes.
 *
 * Conventions for every call:
 *  - Pointers named as device pointers must be device memory (or memory the
 *    device can access); host pointers are read before the call returns.
 *  - The caller owns and allocates every buffer (the recurrent state's
 *    lifecycle -- retain, reuse, zero, evict -- is the caller's: page
 *    "Qwen3.8-Flash-Next and GLM-5.3-Flash share a 3:1 long-context pattern",
 *    section "Recurrent state and sparse caches need lifecycle controls").
 *    The library allocates no device memory and keeps no pointer after a call
 *    returns.
 *  - Work is enqueued on `hip_stream` (a hipStream_t; NULL = the null stream)
 *    and the call returns without synchronising.  Buffers must stay valid
 *    until the stream has executed the work.
 *  - Every argument is validated on the host before anything is enqueued; a
 *    call that returns an error has enqueued nothing.  No call aborts or
 *    throws.  gdr_last_error() gives a message for the last failure on the
 *    calling thread.
 *  - Results are bitwise deterministic run to run (no floating-point atomics).
 *  - Inputs must be finite; log_alpha must be finite (a hard reset with
 *    log_alpha = -inf is not supported).  These preconditions are not checked
 *    (checking would need device reads).
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDR_ABI_VERSION 6

/* The enumerations travel as 32-bit ints.  Compiled as C++ they name that
 * type, so any int a C caller passes (an invalid one included, which the
 * calls reject) is a value the library may read; C sees plain enums of the
 * same size. */
#ifdef __cplusplus
#define GDR_ENUM_BASE : int32_t
#else
#define GDR_ENUM_BASE
#endif

typedef enum gdr_status GDR_ENUM_BASE {
    GDR_SUCCESS = 0,
    GDR_ERROR_INVALID_VALUE = 1,        /* null pointer, bad size, misalignment, overlap */
    GDR_ERROR_NOT_SUPPORTED = 2,        /* valid request outside the compiled kernel set */
    GDR_ERROR_INSUFFICIENT_WORKSPACE = 3,
    GDR_ERROR_LAUNCH_FAILED = 4         /* the HIP runtime refused a launch */
} gdr_status;

typedef enum gdr_dtype GDR_ENUM_BASE {
    GDR_F32 = 0,
    GDR_BF16 = 1
} gdr_dtype;

typedef enum gdr_gate GDR_ENUM_BASE {
    GDR_GATE_HEAD = 0,      /* Gated DeltaNet: log_alpha has one value per (token, head)        */
    GDR_GATE_CHANNEL = 1    /* Kimi Delta Attention: one value per (token, head, key channel)   */
} gdr_gate;

/*
 * Problem shape of a prefill call.
 *  Dense batch:  batch = B sequences of seqlen tokens each, num_seqs = B,
 *                cu_seqlens = NULL.
 *  Packed batch: batch = 1, seqlen = total tokens, num_seqs = N and
 *                cu_seqlens[N+1] gives each sequence's token range.
 *  num_heads is the number of value heads: one state, one write strength and
 *  one decay per value head.  num_qk_heads query-key heads are shared by
 *  groups of G = num_heads / num_qk_heads consecutive value heads: value head
 *  h reads q and k of head h / G (page "How the New Flash Models Work...",
 *  section "The two stacks, layer by layer": the Gated DeltaNet layers have
 *  16 key heads and 48 value heads; the state-size table counts one state per
 *  value head).  num_qk_heads = 0 means num_heads (no grouping).
 */
typedef struct gdr_prefill_shape {
    int32_t batch;
    int32_t seqlen;
    int32_t num_heads;
    int32_t head_dim_k;
    int32_t head_dim_v;
    int32_t num_seqs;
    int32_t num_qk_heads;
} gdr_prefill_shape;

/*
 * Bytes of device workspace gdr_prefill_chunked needs for this problem:
 *  - packed batches (packed != 0, i.e. cu_seqlens will be passed): the
 *    per-call sequence schedule, 2 x 4 x (num_seqs + 1) bytes, rounded up;
 *  - one record per chunk slot and head holding that chunk's state-independent
 *    operands (decayed keys and queries, the transposed end-of-chunk keys, the
 *    UT-transform inverse and the intra-chunk query-key matrix), R bytes each:
 *    (3 C d_k + 2 C^2) x (2 for bf16 q/k/v, 4 for fp32) plus the chunk's decay
 *    (4 d_k or 16 bytes), rounded up to 256.  Chunk slots: ceil(seqlen / C) +
 *    num_seqs (packed) or batch x ceil(seqlen / C) (dense).
 * This is the size for one pass over all chunks, the fastest schedule.  A
 * dense batch also accepts a smaller workspace: the prefill then runs in
 * segments of S >= 16 chunks (the largest S that fits), needing
 * batch x S x num_heads x R bytes of records plus the state carried between
 * segments (num_seqs x num_heads x head_dim_v x head_dim_k x 4 bytes), each
 * part rounded up to 256 bytes.
 * gate, qkv_dtype and chunk_size are the values that will be passed to
 * gdr_prefill_chunked (chunk_size 0 = automatic).  Returns 0 for a NULL shape
 * or an invalid argument.
 */
size_t gdr_prefill_workspace_bytes(const gdr_prefill_shape *shape, gdr_gate gate, gdr_dtype qkv_dtype,
                                   int32_t chunk_size, int32_t packed);

/*
 * Chunked prefill: runs the recurrence over every token of every sequence and
 * writes all outputs and each sequence's final state.
 *
 * Arguments (device pointers unless noted; row-major, contiguous):
 *  shape          host pointer, see gdr_prefill_shape.
 *  gate           GDR_GATE_HEAD or GDR_GATE_CHANNEL.
 *  qkv_dtype      dtype of q, k and v: GDR_BF16 or GDR_F32.
 *  gate_dtype     dtype of beta and log_alpha (both the same): GDR_F32 or
 *                 GDR_BF16.
 *  out_dtype      dtype of out: GDR_F32 or GDR_BF16 (independent of q/k/v;
 *                 bf16 outputs are rounded to nearest even from fp32).
 *  q, k           [batch, seqlen, num_qk_heads, head_dim_k]
 *  v              [batch, seqlen, num_heads, head_dim_v]
 *  beta           [batch, seqlen, num_heads]           write strengths (any finite value)
 *  log_alpha      [batch, seqlen, num_heads]           (GDR_GATE_HEAD)
 *                 [batch, seqlen, num_heads, head_dim_k] (GDR_GATE_CHANNEL)
 *  initial_state  [num_seqs, num_heads, head_dim_v, head_dim_k] fp32, or NULL
 *                 for zeros.
 *  cu_seqlens     NULL (dense) or int32 [num_seqs+1]: 0 = cu[0] <= cu[1] <=
 *                 ... <= cu[N] = seqlen (not checked: device memory).  Empty
 *                 sequences are allowed (their final state = initial state).
 *  chunk_size     tokens per chunk: 0 = automatic (32 where compiled, else 16),
 *                 else one of the compiled sizes below.
 *  dv_slice       value channels one workgroup owns: 0 = automatic, else a
 *                 compiled width below that divides head_dim_v.
 *                 Compiled (q/k/v dtype: head_dim_k; chunk_size; dv_slice):
 *                   bf16: {32, 64, 128}; 32 or 64; 16 or 32
 *                   bf16: 128; 32; 64
 *                   fp32: {16, 32, 64, 128}; 16 or 32; 16
 *                 Any other request returns GDR_ERROR_NOT_SUPPORTED.
 *  scale          readout factor (1 for the printed equations).
 *  out            [batch, seqlen, num_heads, head_dim_v], dtype out_dtype.
 *                 Must not overlap any input.
 *  final_state    [num_seqs, num_heads, head_dim_v, head_dim_k] fp32, or NULL
 *                 (not written).  May equal initial_state (updated in place)
 *                 but must not partially overlap it or any other buffer.
 *  workspace      device buffer of at least gdr_prefill_workspace_bytes(...)
 *                 bytes (may be NULL when that is 0), 256-byte aligned.
 *  hip_stream     hipStream_t to enqueue on.
 * Limits: head_dim_k in {16, 32, 64, 128} (bf16: {32, 64, 128}); head_dim_v
 * a multiple of 16 up to 256; num_heads a multiple of num_qk_heads (when
 * that is not 0); the q/k/v/out/state base pointers 16-byte
 * aligned; beta 4-byte aligned; log_alpha 16-byte aligned for
 * GDR_GATE_CHANNEL, else 4-byte aligned (halved for bf16 gates).  Per-channel
 * decay: the log-decay summed over one chunk must stay above about -170 in
 * every channel (the chunk's operands are scaled around its midpoint in fp32
 * range).
 * Operand range (bf16 q/k/v): v, the state and the intra-chunk update U enter
 * the MFMA products as fp16.  Every |v| and every element of the state along
 * the sequence must stay below 65504 (fp16's largest finite value; beyond it
 * results become inf), and the RMS of v and of the state at or above about
 * 1e-4 (fp16 numbers below 6.1e-5 are subnormal and lose relative precision:
 * at RMS 1e-5 the error reaches several percent of RMS).  Measured within
 * these bounds: out within about 1e-2 RMS of the exact recurrence.  fp32
 * q/k/v carry everything in fp32 and have no such bound.
 * Work: one kernel computes every chunk's record into the workspace, a second
 * walks each sequence's chunks in order (per segment, when the workspace is
 * smaller than gdr_prefill_workspace_bytes reports); all on hip_stream.
 * Returns GDR_SUCCESS or an error status (nothing enqueued on error).
 */
gdr_status gdr_prefill_chunked(const gdr_prefill_shape *shape, gdr_gate gate,
                               gdr_dtype qkv_dtype, gdr_dtype gate_dtype, gdr_dtype out_dtype,
                               const void *q, const void *k, const void *v,
                               const void *beta, const void *log_alpha,
                               const float *initial_state, const int32_t *cu_seqlens,
                               int32_t chunk_size, int32_t dv_slice, float scale,
                               void *out, float *final_state,
                               void *workspace, size_t workspace_bytes,
                               void *hip_stream);

/*
 * gdr_prefill_chunked without a caller-provided workspace, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  The caller still passes every
 * input and output; the workspace is instead a fixed 64 MiB array that the
 * library holds on each GPU it runs on until the process ends.  No call
 * allocates or frees device memory.
 * Arguments, layouts, limits and results: as gdr_prefill_chunked.  A dense
 * batch whose one-pass workspace exceeds 64 MiB runs in segments that fit; a
 * problem whose smallest workspace (always the one-pass size for packed
 * batches) exceeds 64 MiB returns GDR_ERROR_INSUFFICIENT_WORKSPACE, with the
 * sizes in gdr_last_error(), and enqueues nothing.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (the kernels need nothing of it cleared): calls that overlap on
 * one GPU (on different streams, or from different threads without ordering)
 * race and give undefined results.  Calls on one stream are ordered.
 */
gdr_status gdr_prefill_chunked_static(const gdr_prefill_shape *shape, gdr_gate gate,
                                      gdr_dtype qkv_dtype, gdr_dtype gate_dtype, gdr_dtype out_dtype,
                                      const void *q, const void *k, const void *v,
                                      const void *beta, const void *log_alpha,
                                      const float *initial_state, const int32_t *cu_seqlens,
                                      int32_t chunk_size, int32_t dv_slice, float scale,
                                      void *out, float *final_state, void *hip_stream);

/*
 * Decode step: one new token for each of num_seqs sequences.  Reads each
 * (sequence, head) state once, applies the decay, the erase-then-write update
 * and the readout, and writes the state back in place.
 *
 *  num_heads     value heads (states, gates, v, out); num_qk_heads query-key
 *                heads shared by groups of value heads as in gdr_prefill_shape
 *                (0 = num_heads)
 *  q, k       [num_seqs, num_qk_heads, head_dim_k] dtype qkv_dtype
 *  v          [num_seqs, num_heads, head_dim_v]   dtype qkv_dtype
 *  beta       [num_seqs, num_heads]               dtype gate_dtype
 *  log_alpha  [num_seqs, num_heads] (GDR_GATE_HEAD) or
 *             [num_seqs, num_heads, head_dim_k] (GDR_GATE_CHANNEL), dtype
 *             gate_dtype (GDR_F32 or GDR_BF16, the same as beta)
 *  state      [num_seqs, num_heads, head_dim_v, head_dim_k] fp32, read and
 *             written in place (must not overlap any other argument)
 *  out        [num_seqs, num_heads, head_dim_v]   dtype out_dtype (GDR_F32 or
 *             GDR_BF16, rounded to nearest even)
 * Limits: head_dim_k in {16, 32, 64, 128}; head_dim_v a multiple of 4 up to
 * 256; base pointers 16-byte aligned (gates aligned to their element size).
 */
gdr_status gdr_decode_step(int32_t num_seqs, int32_t num_heads, int32_t num_qk_heads, int32_t head_dim_k,
                           int32_t head_dim_v, gdr_gate gate, gdr_dtype qkv_dtype,
                           gdr_dtype gate_dtype, gdr_dtype out_dtype, const void *q, const void *k,
                           const void *v, const void *beta, const void *log_alpha,
                           float *state, float scale, void *out, void *hip_stream);

/*
 * Multi-token decode: up to max_tokens new tokens for each of num_seqs
 * sequences whose states live in a pool of slots.  For the speculative
 * decoding both models serve with (page "How the New Flash Models Work...",
 * section "Decoding several tokens per pass": a draft of several tokens is
 * verified in one pass of the main model) and the replay of accepted tokens
 * that the GLM serving stack names (page "Qwen3.8-Flash-Next and GLM-5.3-Flash
 * share a 3:1 long-context pattern", section "GLM's serving design is
 * explicitly disaggregated": ReplaySSM).
 *
 * For sequence n with slot s = state_slots[n] (n when state_slots is NULL),
 * T_n = num_tokens[n] (max_tokens when NULL) and C_n = num_commit[n] (T_n
 * when NULL), the call runs the recurrence over tokens 0 .. T_n - 1 starting
 * from state_pool[s], writes out[n, t] for every t < T_n, and stores back
 * into state_pool[s] the state after the first C_n tokens only:
 *   C_n = T_n        plain multi-token decode;
 *   C_n = 0          verify a draft: outputs only, the slot is not written;
 *   0 < C_n < T_n    replay the C_n tokens accepted in the previous step, then
 *                    verify a new draft, with one read and one write of the
 *                    state (the caller ignores the replayed tokens' outputs).
 * Device values out of range are clamped, not rejected (they cannot be read
 * on the host): T_n to [0, max_tokens], C_n to [0, T_n]; a sequence whose slot
 * is negative or >= num_slots is skipped (nothing read or written, its outputs
 * left as they were), which is how padding entries of a batch are marked.
 * Two sequences of one call must not share a slot (their updates would race).
 *
 *  q, k         [num_seqs, max_tokens, num_qk_heads, head_dim_k]  qkv_dtype
 *  v            [num_seqs, max_tokens, num_heads, head_dim_v]     qkv_dtype
 *  beta         [num_seqs, max_tokens, num_heads]                 gate_dtype
 *  log_alpha    [num_seqs, max_tokens, num_heads] (GDR_GATE_HEAD) or
 *               [num_seqs, max_tokens, num_heads, head_dim_k]     gate_dtype
 *               (gate_dtype GDR_F32 or GDR_BF16, the same for both)
 *  num_tokens, num_commit, state_slots   int32 [num_seqs] device arrays or NULL
 *  state_pool   [num_slots, num_heads, head_dim_v, head_dim_k] fp32, read and
 *               written in place (must not overlap any other argument)
 *  out          [num_seqs, max_tokens, num_heads, head_dim_v]  out_dtype;
 *               rows t >= T_n are not written
 * Limits: as gdr_decode_step; 1 <= max_tokens <= 64.
 */
gdr_status gdr_decode_tokens(int32_t num_seqs, int32_t max_tokens, int32_t num_heads, int32_t num_qk_heads,
                             int32_t head_dim_k, int32_t head_dim_v, gdr_gate gate, gdr_dtype qkv_dtype,
                             gdr_dtype gate_dtype, gdr_dtype out_dtype, const void *q, const void *k,
                             const void *v, const void *beta, const void *log_alpha,
                             const int32_t *num_tokens, const int32_t *num_commit,
                             const int32_t *state_slots, float *state_pool, int32_t num_slots,
                             float scale, void *out, void *hip_stream);

/*
 * Layer prologue: the steps between a linear-attention layer's input
 * projections and the recurrence, in one pass (page "Qwen3.8-Flash-Next and
 * GLM-5.3-Flash share a 3:1 long-context pattern", section "Kimi Delta
 * Attention extends recurrent memory control": a short convolution of kernel
 * four; page "How the New Flash Models Work...", section "Serving: prefill and
 * decode are different problems": the convolution state travels with the
 * recurrent state from prefill to decode).  The pages name no activation, no
 * normalisation and no gate parameterisation; the flags make the two common
 * choices available and the gates are the write strength and decay in their
 * plainest form.
 *
 * x holds, per token, the C = 2 Hk dk + H dv projected channels: q (Hk heads
 * of dk), then k (Hk x dk), then v (H x dv).  For every channel c and token t
 * of a sequence:
 *     y_t[c] = sum_{j<4} w[c][j] x_{t-3+j}[c]      (causal, per channel)
 * where the three inputs before a sequence's first token are its convolution
 * state (zeros when conv_state_in is NULL); then
 *     y <- y * sigmoid(y)                  if flags & GDR_PROLOGUE_SILU
 *     q, k <- y / |y| per head (over dk)   if flags & GDR_PROLOGUE_QK_NORM
 *                                          (a zero vector stays zero)
 * and q, k, v <- y in x's dtype (bf16: rounded to nearest even).  Gates:
 *     beta = sigmoid(b_logit),  log_alpha = -softplus(a_logit)  (fp32),
 * so alpha = exp(log_alpha) lies in (0, 1).  The new convolution state of each
 * sequence is its last three inputs (older state rows when it has fewer than
 * three tokens).  With seqlen = 1 and batch = num_seqs the call is the decode
 * step's prologue.
 *
 *  shape          as for gdr_prefill_chunked (dense batch or packed by cu_seqlens)
 *  x              [batch, seqlen, C]         bf16 or fp32 (x_dtype)
 *  conv_weight    [C, 4] fp32: tap j multiplies x_{t-3+j}
 *  conv_state_in  [num_seqs, 3, C] x_dtype, or NULL (zeros); row r holds the
 *                 input 3 - r tokens before the sequence's first
 *  conv_state_out [num_seqs, 3, C] x_dtype, or NULL (not written); may equal
 *                 conv_state_in (updated in place)
 *  cu_seqlens     NULL (dense) or int32 [num_seqs + 1]
 *  a_logit        [batch, seqlen, H] (GDR_GATE_HEAD) or [batch, seqlen, H, dk]   fp32
 *  b_logit        [batch, seqlen, H]                                               fp32
 *  q, k           [batch, seqlen, Hk, dk]   out, x_dtype
 *  v              [batch, seqlen, H, dv]    out, x_dtype
 *  beta, log_alpha  out, fp32, shaped as b_logit and a_logit
 * Limits: head_dim_k in {16, 32, 64, 128}; head_dim_v a multiple of 8;
 * x, states, q, k, v and conv_weight 16-byte aligned.  Outputs must not
 * overlap any input or each other.
 */
#define GDR_PROLOGUE_SILU 1
#define GDR_PROLOGUE_QK_NORM 2
gdr_status gdr_layer_prologue(const gdr_prefill_shape *shape, gdr_gate gate, gdr_dtype x_dtype, const void *x,
                              const float *conv_weight, const void *conv_state_in, void *conv_state_out,
                              const int32_t *cu_seqlens, int32_t flags, const float *a_logit, const float *b_logit,
                              void *q, void *k, void *v, float *beta, float *log_alpha, void *hip_stream);

/*
 * Decode step with the layer prologue fused in: one new token for each of
 * num_seqs sequences, given as its projected channels x rather than as q, k,
 * v and gates.  The result is that of gdr_layer_prologue with seqlen = 1
 * (batch = num_seqs, dense) followed by gdr_decode_step on its outputs, except
 * that q, k, v and the gates stay fp32 on the chip in between (the two calls
 * store q, k, v in x_dtype): they never reach device memory (page
 * "Qwen3.8-Flash-Next and GLM-5.3-Flash share a 3:1 long-context pattern",
 * section "Kimi Delta Attention extends recurrent memory control": the short
 * convolution in front of the recurrence; page "How the New Flash Models
 * Work...", section "Serving: prefill and decode are different problems": the
 * convolution state travels with the recurrent state).
 *
 *  num_heads, num_qk_heads, head_dim_k, head_dim_v, gate   as gdr_decode_step
 *  x_dtype        dtype of x and of the convolution states: GDR_BF16 or GDR_F32
 *  out_dtype      dtype of out: GDR_F32 or GDR_BF16
 *  x              [num_seqs, C], C = 2 num_qk_heads head_dim_k + num_heads
 *                 head_dim_v: q, k, v channels as for gdr_layer_prologue
 *  conv_weight    [C, 4] fp32 (tap j multiplies x_{t-3+j})
 *  conv_state_in  [num_seqs, 3, C] x_dtype, or NULL (zeros)
 *  conv_state_out [num_seqs, 3, C] x_dtype, or NULL (not written); may equal
 *                 conv_state_in (advanced in place)
 *  flags          GDR_PROLOGUE_SILU | GDR_PROLOGUE_QK_NORM, as for
 *                 gdr_layer_prologue
 *  a_logit        [num_seqs, num_heads] (GDR_GATE_HEAD) or
 *                 [num_seqs, num_heads, head_dim_k] fp32: log_alpha = -softplus(a)
 *  b_logit        [num_seqs, num_heads] fp32: beta = sigmoid(b)
 *  state          [num_seqs, num_heads, head_dim_v, head_dim_k] fp32, read and
 *                 written in place
 *  out            [num_seqs, num_heads, head_dim_v], dtype out_dtype
 * Limits: head_dim_k in {16, 32, 64, 128}; head_dim_v a multiple of 8 up to
 * 256; x, the convolution states, conv_weight and state 16-byte aligned (and
 * a_logit for GDR_GATE_CHANNEL), other gates 4-byte aligned.  state, out and
 * conv_state_out must not overlap the inputs or each other (except
 * conv_state_out == conv_state_in).
 * Work: one kernel for the prologue and the state update, a second small one
 * that advances the convolution state (after the first on hip_stream, so the
 * in-place update is safe).  Returns GDR_SUCCESS or an error status (nothing
 * enqueued on error).
 */
gdr_status gdr_decode_step_prologue(int32_t num_seqs, int32_t num_heads, int32_t num_qk_heads, int32_t head_dim_k,
                                    int32_t head_dim_v, gdr_gate gate, gdr_dtype x_dtype, gdr_dtype out_dtype,
                                    const void *x, const float *conv_weight, const void *conv_state_in,
                                    void *conv_state_out, int32_t flags, const float *a_logit, const float *b_logit,
                                    float *state, float scale, void *out, void *hip_stream);

/* Bytes of fp32 recurrent state for num_seqs x num_heads heads of d_v x d_k
 * (the per-layer state the pages size in their state-size table). */
uint64_t gdr_state_bytes(int64_t num_seqs, int64_t num_heads, int64_t head_dim_k, int64_t head_dim_v);

/* Static description of a status code. */
const char *gdr_status_string(gdr_status status);

/*
 * Backward of gdr_prefill_chunked, for training.  The recurrence is the one
 * of page "How the New Flash Models Work: Inside GLM-5.3-Flash and
 * Qwen3.8-Flash-Next", section "Linear attention: a fixed-size memory in
 * place of the cache" (Gated DeltaNet and Kimi Delta Attention equations);
 * the pages train these layers but give no backward pass, so this is the
 * chain rule of the forward computation.  Given the gradients of a scalar
 * loss with respect to the forward's outputs (d_out) and final states
 * (d_final_state), it returns the loss's gradients with respect to q, k, v,
 * beta, log_alpha and the initial state.  The forward's outputs are not
 * needed: the chunks' states are recomputed.
 *
 *  shape, gate, qkv_dtype, gate_dtype, q, k, v, beta, log_alpha,
 *                 initial_state, cu_seqlens, scale
 *                 exactly as passed to gdr_prefill_chunked (grouped q/k
 *                 heads and bf16 gates included).
 *  d_out          [batch, seqlen, num_heads, head_dim_v]              fp32
 *  d_final_state  [num_seqs, num_heads, head_dim_v, head_dim_k] fp32, or
 *                 NULL for zeros
 *  dq, dk         [batch, seqlen, num_qk_heads, head_dim_k]           fp32
 *                 (a shared q/k head's gradient sums its value heads')
 *  dv             [batch, seqlen, num_heads, head_dim_v]              fp32
 *  dbeta          [batch, seqlen, num_heads]                          fp32
 *  dlog_alpha     log_alpha's shape                                   fp32
 *                 (fp32 also for bf16 gates)
 *  d_initial_state [num_seqs, num_heads, head_dim_v, head_dim_k] fp32, or
 *                 NULL (not written).  With a NULL initial_state it is the
 *                 gradient with respect to the zero state.
 *  workspace      device buffer of gdr_prefill_backward_workspace_bytes(...)
 *                 bytes, 256-byte aligned; the library writes it (chunk
 *                 records, each chunk's state and state gradient: about
 *                 1.8 KB + 8 d_k d_v / 32 bytes, 5.9 KB at d = 128, per token
 *                 and value head; with grouped q/k heads also the value
 *                 heads' dq and dk) and keeps nothing in it after the stream
 *                 has run the call.  That is one pass over all chunks, the
 *                 fastest schedule.  A dense batch also accepts a smaller
 *                 workspace, down to
 *                 gdr_prefill_backward_segment_workspace_bytes(shape, gate, 16):
 *                 the call then runs in the fewest time segments that fit,
 *                 NS of them with S = max(16, ceil(chunks per sequence / NS))
 *                 chunks each (the last one shorter), keeping records and per-chunk states
 *                 for one segment only, plus the state entering each later
 *                 segment and two state gradients carried between segments.
 *                 A first forward pass over the segments finds those states;
 *                 each segment's records and forward states are then built
 *                 again, so the call takes longer.  The results are the same
 *                 bit for bit.  Packed batches need the one-pass size.
 *
 * Supported: head_dim_k in {32, 64, 128}; head_dim_v in {32, 64, 96, 128}
 * (else GDR_ERROR_NOT_SUPPORTED).  q, k, v, d_out, dq, dk and the states
 * 16-byte aligned; beta aligned to its element, log_alpha to four elements
 * for GDR_GATE_CHANNEL; the other gradients 4-byte.  No output may overlap an input, another output or the
 * workspace.  Data and accumulation are fp32; the products with a head_dim
 * contraction take their operands as bf16 hi + lo pairs (16 significant
 * bits, relative error about 2^-16 per product).  Every gradient element is
 * written by exactly one thread (no atomics), so results are bitwise
 * reproducible.
 * Rows of padding and packed sequences of length zero are handled (an empty
 * sequence's d_initial_state is its d_final_state).  Enqueued on hip_stream;
 * returns GDR_SUCCESS or an error status (nothing enqueued on error).
 */
size_t gdr_prefill_backward_workspace_bytes(const gdr_prefill_shape *shape, gdr_gate gate, int32_t packed);
/* Workspace of gdr_prefill_backward for a dense batch (cu_seqlens NULL) run in
 * time segments of segment_chunks chunks of 32 tokens: for
 * NS = ceil(ceil(seqlen / 32) / segment_chunks) segments, batch x
 * segment_chunks x num_heads records and state pairs, plus (NS - 1 + 2) x
 * num_seqs x num_heads x head_dim_v x head_dim_k x 4 bytes of states carried
 * between segments, each part rounded up to 256 bytes (and the grouped
 * heads' dq, dk as in one pass).  With segment_chunks at or above the chunks
 * per sequence it is the one-pass size.  Returns 0 for a NULL shape, an
 * invalid gate or segment_chunks below 16. */
size_t gdr_prefill_backward_segment_workspace_bytes(const gdr_prefill_shape *shape, gdr_gate gate,
                                                    int32_t segment_chunks);
gdr_status gdr_prefill_backward(const gdr_prefill_shape *shape, gdr_gate gate, gdr_dtype qkv_dtype,
                                gdr_dtype gate_dtype, const void *q, const void *k, const void *v, const void *beta,
                                const void *log_alpha, const float *initial_state, const int32_t *cu_seqlens,
                                float scale, const float *d_out, const float *d_final_state, float *dq,
                                float *dk, float *dv, float *dbeta, float *dlog_alpha, float *d_initial_state,
                                void *workspace, size_t workspace_bytes, void *hip_stream);

/* Detail of the last failing call on the calling thread ("" if none). */
const char *gdr_last_error(void);

/* GDR_ABI_VERSION of the built library. */
int gdr_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */

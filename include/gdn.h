/*
 * gdn.h - C ABI of the Gated DeltaNet recurrence library for AMD MI355X
 * (gfx950).
 *
 * The operation.  Each value head keeps a fixed d x d memory matrix S
 * (page "Inside Qwen3.8-27B: Hybrid DeltaNet Architecture, 256k Context, and
 * 24GB Local Serving", section "Gated DeltaNet Mechanics": a delta rule that
 * erases the current association of a normalized key before writing the new
 * value, under a per-token decay, with a state whose size does not depend on
 * the context length).  The page's update formula is missing from its text;
 * the library computes the gated delta rule that has every property the page
 * lists:
 *
 *     S_t = alpha_t * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t                                   (state after the update)
 *
 * Shapes follow the 27B model's DeltaNet layers (page "Qwen 3.8 27B Review:
 * Native Vision, FP8 Quantization & 1M Context in a Compact Dense Model",
 * section 3): 16 query/key heads, 48 value heads, head dim 128.  Value head h
 * reads query/key head h / (H_v / H_qk): contiguous groups of H_v / H_qk value
 * heads share one query/key head.  Only D = 128 is supported.
 *
 * Prefill uses the block-parallel (chunked) form of the same recurrence (same
 * page as above, the note under "The Role of Periodic Gated Attention"), 64
 * tokens per chunk: an in-chunk triangular (UT) solve and a serial carry of the
 * state from chunk to chunk, with the state resident on chip.  Decode advances
 * every sequence by one token (same note: sequential at inference).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers of the current HIP device,
 *    contiguous, row-major, in the layouts given per call.  q, k, v, o and
 *    gate have the element type `dt`; alpha, beta, states (h0, ht, state) and
 *    norm_weight are always float32.
 *  - State layout [.., H_v, D, D]: row = value index, column = key index
 *    (S is d_v x d_k), so one value row is D contiguous floats.
 *  - q and k are expected L2-normalised per (token, head) by the caller;
 *    alpha in (0, 1], beta in [0, 1].  These are preconditions (not checked):
 *    alpha = 0 is not supported (the chunked form works with log(alpha)).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on that stream and returns; it never allocates, frees or
 *    synchronises.  Device faults surface at the caller's next synchronisation.
 *  - The caller owns every buffer, including the workspace; the library keeps
 *    no global mutable state, so calls from several host threads are safe.
 *    The one exception is gdn_prefill_chunked_noalloc, whose workspace is a
 *    static array of the library (see there).
 *  - Every argument check runs on the host before anything is enqueued: a
 *    call that returns an error has enqueued nothing.
 *  - Pointers must be 16-byte aligned (alpha, beta: 4-byte).  Outputs must not
 *    overlap inputs, except that `ht` may be exactly `h0` (in-place carry).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v, o and gate: GDN_F32 or GDN_BF16.  A plain integer
 * rather than an enum, so that any value a caller passes is well defined on
 * the library side (an unknown one returns GDN_ERR_UNSUPPORTED). */
typedef int32_t gdn_dtype;
#define GDN_F32 0
#define GDN_BF16 1

typedef int gdn_status;
#define GDN_OK 0
#define GDN_ERR_NULL (-1)        /* a required pointer is NULL               */
#define GDN_ERR_SHAPE (-2)       /* negative or inconsistent sizes          */
#define GDN_ERR_UNSUPPORTED (-3) /* D != 128, unknown dtype, size overflow  */
#define GDN_ERR_ALIGN (-4)       /* a pointer is not aligned                */
#define GDN_ERR_ALIAS (-5)       /* an output overlaps another buffer       */
#define GDN_ERR_WORKSPACE (-6)   /* workspace missing or too small          */
#define GDN_ERR_HIP (-7)         /* a HIP launch failed; see gdn_last_hip_error */
#define GDN_ERR_TOO_LARGE (-8)   /* needs more than GDN_NOALLOC_SCRATCH_BYTES  */

/* Tokens per chunk of the block-parallel prefill. */
#define GDN_CHUNK 64

/*
 * gdn_prefill_chunked - chunked prefill of B sequences of equal length T.
 *
 *   q, k   [B, T, H_qk, D]  dt
 *   v      [B, T, H_v, D]   dt
 *   alpha  [B, T, H_v]      float32   per-token decay of the state
 *   beta   [B, T, H_v]      float32   per-token write strength
 *   h0     [B, H_v, D, D]   float32   initial state, or NULL for zeros
 *   o      [B, T, H_v, D]   dt        output o_t = S_t q_t
 *   ht     [B, H_v, D, D]   float32   final state, or NULL (not written);
 *                                     may be exactly h0
 *   workspace, workspace_bytes: at least gdn_prefill_workspace_bytes(...)
 *                                     bytes of device memory, contents
 *                                     ignored on entry and clobbered
 * T = 0 is allowed: then ht receives h0 (or zeros).  The state size, and so
 * h0/ht, does not depend on T.
 */
gdn_status gdn_prefill_chunked(const void *q, const void *k, const void *v,
                               const float *alpha, const float *beta,
                               const float *h0, void *o, float *ht,
                               int32_t B, int32_t T, int32_t H_qk, int32_t H_v,
                               int32_t D, gdn_dtype dt, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * gdn_prefill_chunked_noalloc - gdn_prefill_chunked without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 *
 * Same arguments, layouts, results and errors as gdn_prefill_chunked, minus
 * workspace/workspace_bytes.  The workspace is a static device array of the
 * library, GDN_NOALLOC_SCRATCH_BYTES (128 MiB) per GPU, held from the
 * library's first use on that GPU until the process ends.  A call whose
 * gdn_prefill_workspace_bytes(...) exceeds it returns GDN_ERR_TOO_LARGE and
 * enqueues nothing (bf16 or fp32 at H_v = 48: B * ceil(T / 64) <= 165 or 84
 * chunks, e.g. one T = 8192 bf16 sequence).  Nothing in the array needs to
 * start at zero; it keeps the last call's contents.
 *
 * Every call on one GPU uses that GPU's single array: calls whose execution
 * overlaps on one GPU (different streams, or host threads racing on
 * different streams) race on it and give wrong results.  Serialise them, e.g.
 * by using one stream per GPU.  The first call on a GPU looks up the array's
 * device address (hipGetSymbolAddress), which neither allocates nor
 * synchronises.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
gdn_status gdn_prefill_chunked_noalloc(const void *q, const void *k,
                                       const void *v, const float *alpha,
                                       const float *beta, const float *h0,
                                       void *o, float *ht, int32_t B,
                                       int32_t T, int32_t H_qk, int32_t H_v,
                                       int32_t D, gdn_dtype dt, void *stream);

/* Workspace bytes for gdn_prefill_chunked (0 on unsupported arguments).
 * Grows with the number of chunks (per-chunk solve results), never with the
 * state. */
size_t gdn_prefill_workspace_bytes(int32_t B, int32_t T, int32_t H_qk,
                                   int32_t H_v, int32_t D, gdn_dtype dt);

/*
 * The two stream-ordered halves of gdn_prefill_chunked, same arguments.
 * gdn_prefill_prepare runs the fully parallel in-chunk part (gate prefix,
 * Gram matrices, triangular solve) into the workspace; gdn_prefill_scan runs
 * the serial inter-chunk state carry and the outputs from it.  Calling
 * prepare then scan on one stream with one workspace is exactly
 * gdn_prefill_chunked.  They exist so that each half can be timed alone.
 */
gdn_status gdn_prefill_prepare(const void *q, const void *k, const void *v,
                               const float *alpha, const float *beta,
                               const float *h0, void *o, float *ht,
                               int32_t B, int32_t T, int32_t H_qk, int32_t H_v,
                               int32_t D, gdn_dtype dt, void *workspace,
                               size_t workspace_bytes, void *stream);
gdn_status gdn_prefill_scan(const void *q, const void *k, const void *v,
                            const float *alpha, const float *beta,
                            const float *h0, void *o, float *ht,
                            int32_t B, int32_t T, int32_t H_qk, int32_t H_v,
                            int32_t D, gdn_dtype dt, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * gdn_decode_step - one token for each of B sequences, state updated in place
 * (page "Inside Qwen3.8-27B ...", note under "The Role of Periodic Gated
 * Attention": at inference the state advances one token at a time).
 *
 *   q, k   [B, H_qk, D]     dt
 *   v      [B, H_v, D]      dt
 *   alpha, beta [B, H_v]    float32
 *   state  [B, H_v, D, D]   float32, read and overwritten with S_t
 *   o      [B, H_v, D]      dt
 * No workspace.  The update is not transactional: a caller that may need
 * the previous state keeps a copy.
 */
gdn_status gdn_decode_step(const void *q, const void *k, const void *v,
                           const float *alpha, const float *beta, float *state,
                           void *o, int32_t B, int32_t H_qk, int32_t H_v,
                           int32_t D, gdn_dtype dt, void *stream);

/*
 * States stored as bfloat16.  The pages count the recurrent-state footprint
 * at BF16 (page "Qwen3.8 Explained: 27B Multimodal, 2.4T MoE, and the VRAM
 * Math", section "The architecture detail that matters for VRAM": a constant
 * overhead of tens of megabytes over the 48 DeltaNet layers).  These calls
 * take and return the state in bfloat16; all arithmetic stays fp32, and a
 * state is rounded to bfloat16 (nearest even) only where it is stored.
 *
 * gdn_decode_step_bf16_state: as gdn_decode_step with
 *   state  [B, H_v, D, D]   bfloat16, read and overwritten with S_t
 * which halves the bytes the step moves.  Same errors and aliasing rules.
 */
gdn_status gdn_decode_step_bf16_state(const void *q, const void *k,
                                      const void *v, const float *alpha,
                                      const float *beta, void *state, void *o,
                                      int32_t B, int32_t H_qk, int32_t H_v,
                                      int32_t D, gdn_dtype dt, void *stream);

/*
 * gdn_prefill_chunked_bf16_state: as gdn_prefill_chunked with
 *   h0     [B, H_v, D, D]   bfloat16 initial state, or NULL for zeros
 *   ht     [B, H_v, D, D]   bfloat16 final state, or NULL; may be exactly h0
 * (the carry between a prefill and the decode steps that follow it).  The
 * state inside the call is fp32; only h0 and ht are bfloat16.  Uses the same
 * workspace size as gdn_prefill_chunked.
 */
gdn_status gdn_prefill_chunked_bf16_state(const void *q, const void *k,
                                          const void *v, const float *alpha,
                                          const float *beta, const void *h0,
                                          void *o, void *ht, int32_t B,
                                          int32_t T, int32_t H_qk, int32_t H_v,
                                          int32_t D, gdn_dtype dt,
                                          void *workspace,
                                          size_t workspace_bytes, void *stream);

/*
 * Speculative decoding with drafted tokens (page "Inside Qwen3.8-27B ...",
 * section "Multi-Token Prediction (MTP)": extra heads draft the next tokens,
 * which the model then verifies).  For n drafted tokens per sequence
 * (1 <= n <= 8):
 *
 * gdn_decode_verify: the outputs of all n tokens, token t's output being
 * S_t q_t with S_t the state after tokens 0..t, computed from `state`,
 * which is only read.
 *   q, k   [B, n, H_qk, D]  dt
 *   v      [B, n, H_v, D]   dt
 *   alpha, beta [B, n, H_v] float32
 *   state  [B, H_v, D, D]   float32, not modified
 *   o      [B, n, H_v, D]   dt
 *
 * gdn_decode_commit: advances `state` in place by the first
 * min(max(n_accept[b], 0), n) tokens of sequence b, the accepted prefix (0:
 * unchanged).  n_accept is an int32 DEVICE array [B], so the count decided on
 * the device needs no host round trip.  k, v, alpha, beta as for verify.
 *
 * Verify then commit is the rollback of a rejected draft: the state is never
 * advanced past the accepted prefix, and no snapshot is kept.  Verify reads
 * the state once, and commit reads and writes it once, whatever n is.
 * n > 8 returns GDN_ERR_UNSUPPORTED.
 */
gdn_status gdn_decode_verify(const void *q, const void *k, const void *v,
                             const float *alpha, const float *beta,
                             const float *state, void *o, int32_t B, int32_t n,
                             int32_t H_qk, int32_t H_v, int32_t D, gdn_dtype dt,
                             void *stream);
gdn_status gdn_decode_commit(const void *k, const void *v, const float *alpha,
                             const float *beta, float *state,
                             const int32_t *n_accept, int32_t B, int32_t n,
                             int32_t H_qk, int32_t H_v, int32_t D, gdn_dtype dt,
                             void *stream);

/*
 * gdn_prefill_varlen - N sequences of different lengths packed along the
 * token axis (several concurrent sequences, as a serving engine batches them:
 * page "Inside Qwen3.8-27B ...", section "Serving Qwen3.8-27B: Recipes for
 * vLLM and SGLang").  Each sequence is an independent recurrence from its own
 * initial state; chunks restart at every sequence start.
 *
 *   q, k        [T_tot, H_qk, D]  dt
 *   v           [T_tot, H_v, D]   dt
 *   alpha, beta [T_tot, H_v]      float32
 *   cu_seqlens  [N + 1]           int32 DEVICE pointer: cu_seqlens[0] = 0,
 *                                 non-decreasing, cu_seqlens[N] = T_tot
 *                                 (precondition; never read on the host,
 *                                 except with the environment variable
 *                                 GDN_DEBUG=1: then the call copies it to
 *                                 the host, synchronously on `stream`, and
 *                                 returns GDN_ERR_SHAPE if it is malformed).
 *                                 Zero-length sequences are allowed.
 *   h0          [N, H_v, D, D]    float32 or NULL (zeros)
 *   o           [T_tot, H_v, D]   dt
 *   ht          [N, H_v, D, D]    float32 or NULL; may be exactly h0
 *   gate        [T_tot, H_v, D]   dt or NULL.  When given, o receives
 *                 y = o_t / sqrt(mean_d(o_t^2) + norm_eps) * w * sigmoid(gate)
 *                 per (token, head): an RMS normalisation over the head dim
 *                 (as the card "Qwen3.8 (27B)" describes RMSNorm for QK-Norm)
 *                 followed by a learned sigmoid output gate (as the same card
 *                 describes Gated Attention's output gate).
 *   norm_weight [D] float32 or NULL (all ones); used only with gate.
 *   workspace   at least gdn_varlen_workspace_bytes(...) bytes.
 */
gdn_status gdn_prefill_varlen(const void *q, const void *k, const void *v,
                              const float *alpha, const float *beta,
                              const int32_t *cu_seqlens, int32_t N,
                              int32_t T_tot, const float *h0, void *o,
                              float *ht, const void *gate,
                              const float *norm_weight, float norm_eps,
                              int32_t H_qk, int32_t H_v, int32_t D,
                              gdn_dtype dt, void *workspace,
                              size_t workspace_bytes, void *stream);

/* Workspace bytes for gdn_prefill_varlen.  Sized for ceil(T_tot/64) + N
 * chunks, so the host never needs to read cu_seqlens. */
size_t gdn_varlen_workspace_bytes(int32_t N, int32_t T_tot, int32_t H_qk,
                                  int32_t H_v, int32_t D, gdn_dtype dt);

/*
 * gdn_prefill_chunked_bwd - gradients of gdn_prefill_chunked (training runs
 * the same block-parallel form as prefill: page "Inside Qwen3.8-27B ...", the
 * note under "The Role of Periodic Gated Attention").  For the scalar
 *     L = sum_t <dout_t, o_t> + <dht, S_T>
 * it returns dL/dq, dL/dk, dL/dv, dL/dalpha, dL/dbeta and dL/dh0.
 *
 *   q, k, v, alpha, beta, h0   the forward call's inputs (same layouts; h0
 *                              may be NULL for a zero initial state)
 *   dout   [B, T, H_v, D]   dt        dL/do
 *   dht    [B, H_v, D, D]   float32   dL/dS_T, or NULL (zero)
 *   dq, dk [B, T, H_qk, D]  dt        summed over the value heads sharing
 *                                     each query/key head
 *   dv     [B, T, H_v, D]   dt
 *   dalpha, dbeta [B, T, H_v] float32
 *   dh0    [B, H_v, D, D]   float32   or NULL (not written)
 *   workspace  at least gdn_prefill_bwd_workspace_bytes(...) bytes; it holds
 *              the state entering every chunk and the gradient of the state
 *              leaving every chunk (element type dt), so it grows with T.
 * The forward states are recomputed from the inputs (nothing is kept from the
 * forward call).  Outputs must not overlap inputs, each other or the
 * workspace.  Arithmetic: dt operands on the matrix units, fp32 accumulation
 * and fp32 carried state gradient.  T = 0 gives dh0 = dht (or zeros).
 */
gdn_status gdn_prefill_chunked_bwd(const void *q, const void *k, const void *v,
                                   const float *alpha, const float *beta,
                                   const float *h0, const void *dout,
                                   const float *dht, void *dq, void *dk,
                                   void *dv, float *dalpha, float *dbeta,
                                   float *dh0, int32_t B, int32_t T,
                                   int32_t H_qk, int32_t H_v, int32_t D,
                                   gdn_dtype dt, void *workspace,
                                   size_t workspace_bytes, void *stream);

/* Workspace bytes for gdn_prefill_chunked_bwd (0 on unsupported arguments). */
size_t gdn_prefill_bwd_workspace_bytes(int32_t B, int32_t T, int32_t H_qk,
                                       int32_t H_v, int32_t D, gdn_dtype dt);

/*
 * gdn_prefill_varlen_bwd - gradients of a packed prefill (gdn_prefill_varlen
 * without the gated output): N sequences packed along the token axis with
 * cu_seqlens, as training batches pack them.  Layouts as for
 * gdn_prefill_varlen and gdn_prefill_chunked_bwd with the token axis T_tot:
 * dout, dv [T_tot, H_v, D]; dq, dk [T_tot, H_qk, D]; dalpha, dbeta
 * [T_tot, H_v]; h0, dht, dh0 [N, H_v, D, D] float32 (h0, dht and dh0 may be
 * NULL).  cu_seqlens is the same int32 DEVICE array (precondition: starts at
 * 0, non-decreasing, ends at T_tot; never read on the host).  workspace at
 * least gdn_varlen_bwd_workspace_bytes(...) bytes.
 */
gdn_status gdn_prefill_varlen_bwd(const void *q, const void *k, const void *v,
                                  const float *alpha, const float *beta,
                                  const int32_t *cu_seqlens, int32_t N,
                                  int32_t T_tot, const float *h0,
                                  const void *dout, const float *dht, void *dq,
                                  void *dk, void *dv, float *dalpha,
                                  float *dbeta, float *dh0, int32_t H_qk,
                                  int32_t H_v, int32_t D, gdn_dtype dt,
                                  void *workspace, size_t workspace_bytes,
                                  void *stream);

size_t gdn_varlen_bwd_workspace_bytes(int32_t N, int32_t T_tot, int32_t H_qk,
                                      int32_t H_v, int32_t D, gdn_dtype dt);

/*
 * Gated attention layer: the other layer type of the hybrid stack (one in four
 * layers; page "Inside Qwen3.8-27B ...", section "The Role of Periodic Gated
 * Attention": 24 query heads, 4 key/value heads, head dim 256, rotary
 * embedding on a 64-channel subspace with theta = 10,000,000).  From the
 * projected per-head activations, per (token, head):
 *
 *   q, k <- RMSNorm(q, k) * w      QK-Norm over the 256 channels (card
 *                                  "Qwen3.8 (27B)", "Architecture concepts";
 *                                  w = the norm weight, ones when NULL)
 *   rotate channels (j, j + rope_dim/2), j < rope_dim/2, by the angle
 *          pos * theta^(-2j / rope_dim); channels >= rope_dim pass through
 *   o = softmax_causal(q k^T / sqrt(256)) v      query head h reads key/value
 *                                  head h / (H_q / H_kv)
 *   o <- o * sigmoid(gate)         channel by channel (the output gate that
 *                                  the fused q projection carries: page
 *                                  "Qwen3.8 Explained ...", the note on
 *                                  attn_output_gate)
 *
 * D must be 256, H_q / H_kv <= 8, rope_dim a multiple of 8 in [0, 256],
 * theta > 0, norm_eps >= 0 (else GDN_ERR_UNSUPPORTED or GDN_ERR_SHAPE).  All
 * tensors of dtype dt except the fp32 norm weights; 16-byte aligned (norm
 * weights and pos 4-byte).  Sizes: B * T (prefill) and B * cache_len
 * (decode) at most 2^25, and B * T * (H_q + H_kv) below 2^31, else
 * GDN_ERR_UNSUPPORTED.  Outputs (o, the caches, the workspace) may overlap
 * neither an input nor each other.
 *
 * gdn_attn_prefill - B sequences of T tokens at positions 0 .. T-1.
 *   q, gate   [B, T, H_q, D]   dt
 *   k, v      [B, T, H_kv, D]  dt
 *   o         [B, T, H_q, D]   dt
 *   k_cache, v_cache  [B, cache_len, H_kv, D] dt, both or neither.  When
 *             given (cache_len >= T), rows 0 .. T-1 receive the normalised,
 *             rotated keys and the values, ready for gdn_attn_decode; rows
 *             >= T are untouched.
 *   workspace at least gdn_attn_prefill_workspace_bytes(...) bytes.
 */
gdn_status gdn_attn_prefill(const void *q, const void *k, const void *v,
                            const void *gate, const float *q_norm_w,
                            const float *k_norm_w, float norm_eps, void *o,
                            void *k_cache, void *v_cache, int32_t cache_len,
                            int32_t B, int32_t T, int32_t H_q, int32_t H_kv,
                            int32_t D, int32_t rope_dim, float rope_theta,
                            gdn_dtype dt, void *workspace,
                            size_t workspace_bytes, void *stream);

size_t gdn_attn_prefill_workspace_bytes(int32_t B, int32_t T, int32_t H_q,
                                        int32_t H_kv, int32_t D, gdn_dtype dt);

/*
 * gdn_attn_decode - one new token for each of B sequences.
 *   q, gate   [B, H_q, D]  dt;   k, v [B, H_kv, D] dt;   o [B, H_q, D] dt
 *   pos       [B] int32 DEVICE array: the token's position, i.e. the number
 *             of tokens already in the cache (precondition 0 <= pos[b] <
 *             cache_len; the kernels clamp it into range, never read it on
 *             the host).
 *   k_cache, v_cache [B, cache_len, H_kv, D] dt: row pos[b] receives the
 *             token's normalised, rotated key and its value; the token then
 *             attends to rows 0 .. pos[b].
 *   workspace at least gdn_attn_decode_workspace_bytes(...) bytes: the
 *             rotated queries and one (max, sum, 256-wide sum) partial per
 *             key split and query head; the keys are split so that the grid
 *             holds about two workgroups per CU, so the size depends on B,
 *             H_kv and cache_len.
 * The caller advances pos.
 */
gdn_status gdn_attn_decode(const void *q, const void *k, const void *v,
                           const void *gate, const float *q_norm_w,
                           const float *k_norm_w, float norm_eps, void *o,
                           void *k_cache, void *v_cache, const int32_t *pos,
                           int32_t cache_len, int32_t B, int32_t H_q,
                           int32_t H_kv, int32_t D, int32_t rope_dim,
                           float rope_theta, gdn_dtype dt, void *workspace,
                           size_t workspace_bytes, void *stream);

size_t gdn_attn_decode_workspace_bytes(int32_t B, int32_t cache_len,
                                       int32_t H_q, int32_t H_kv, int32_t D,
                                       gdn_dtype dt);

/* Human-readable name of a status code (static string). */
const char *gdn_status_str(gdn_status s);

/* The hipError_t of the last failed launch on the calling thread (0 if none). */
int gdn_last_hip_error(void);

/* ABI version: 100 * major + minor. */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */

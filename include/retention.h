/* Multi-scale retention (RetNet) for AMD MI355X (gfx950): C ABI.
 *
 * The method: "Retentive Network: A Successor to Transformer for Large
 * Language Models" (Elamur Research summary). Section "Summary": retention
 * replaces attention; it comes from a linear recurrence with exponential
 * decay; positions are encoded like xPos; there are parallel, recurrent and
 * chunkwise forms; every head has its own decay; a swish gate and GroupNorm
 * follow. Section "Key points", fifth item: head i decays with
 * g_i = 1 - 2^(-5-i), and the chunkwise form costs O(dn(b+h)).
 *
 * Per head with decay g, token n of a sequence (0-based) gets
 *     o_n = sum_{m<=n} g^(n-m) (q_n . k_m) v_m + g^(n+1) q_n S0
 * (S0: a carried-in state, zero unless given), equivalently the recurrence
 *     S_n = g S_{n-1} + k_n^T v_n,   o_n = q_n S_n.
 * q and k are first rotated by position: adjacent pairs (2j, 2j+1) turn by
 * (pos_offset + n) * base^(-2j/dk) radians. When a gate G is given the output
 * is GroupNorm(o) (one group per head over its dv values, biased variance, no
 * affine) times swish(G) = G * sigmoid(G).
 *
 * Memory layouts (all row-major, contiguous, caller-owned DEVICE memory):
 *     q, k          [batch, seqlen, heads, dk]     dtype of the descriptor
 *     v, g, o       [batch, seqlen, heads, dv]     dtype of the descriptor
 *     state         [batch, heads, dk, dv]         fp32, always
 * Every pointer must be 16-byte aligned. A buffer a call writes (o, a state
 * it writes, the workspace) must not overlap any other argument
 * (RET_ERR_ALIAS), except state_in == state_out exactly where allowed.
 *
 * Every call validates its arguments on the host first and returns an error
 * status without touching the device when they are invalid. On success it
 * enqueues its kernels on `stream` and returns at once; faults inside the
 * kernels surface at the caller's next synchronisation. The library keeps no
 * pointer after a call returns, allocates no device memory and holds no
 * global mutable state (except the static scratch of
 * retention_chunkwise_fwd_noalloc), so calls on different streams may run
 * concurrently when their buffers (workspace included) are distinct. Results are bitwise
 * deterministic for a given build, shape and input.
 *
 * Supported: dk == dv in {64, 128, 256}; dtype fp32 or bf16; heads <= 128.
 * Arithmetic: bf16 inputs are multiplied on the matrix cores with fp32
 * accumulation; fp32 inputs use fp32 matrix-core products. The state, decay
 * factors, GroupNorm and gate run in fp32.
 */
#ifndef RETENTION_H
#define RETENTION_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RET_OK = 0,
  RET_ERR_NULL = 1,        /* a required pointer is NULL                        */
  RET_ERR_SHAPE = 2,       /* batch, seqlen, heads or chunk out of range        */
  RET_ERR_UNSUPPORTED = 3, /* dk/dv/dtype combination not built                 */
  RET_ERR_GAMMA = 4,       /* a decay outside (0, 1], or not finite             */
  RET_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned                  */
  RET_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required          */
  RET_ERR_HIP = 7,         /* the HIP runtime rejected a kernel launch          */
  RET_ERR_ALIAS = 8,       /* the output overlaps an input                      */
  RET_ERR_ARG = 9,         /* another scalar argument is invalid (eps, base...) */
  RET_ERR_SCRATCH = 10     /* needs more than the static scratch (_noalloc only) */
} ret_status_t;

typedef enum { RET_F32 = 0, RET_BF16 = 1 } ret_dtype_t;

typedef struct {
  int32_t batch;       /* >= 1                                                 */
  int32_t seqlen;      /* >= 1 (exactly 1 for retention_recurrent_step)        */
  int32_t heads;       /* 1 .. 128                                             */
  int32_t dk;          /* query/key head dimension                             */
  int32_t dv;          /* value head dimension (== dk)                         */
  int32_t dtype;       /* ret_dtype_t of q, k, v, g and o                      */
  const double *gamma; /* HOST array [heads] of decays in (0, 1]; NULL selects
                          the per-head default g_i = 1 - 2^(-5-i)               */
  double rotary_base;  /* 0: no rotation; else theta_j = base^(-2j/dk), > 0   */
  int64_t pos_offset;  /* absolute position of token 0 (rotation only), >= 0  */
  float gn_eps;        /* GroupNorm epsilon, > 0; used only when g != NULL    */
} ret_desc_t;

/* Parallel form: O = (Q K^T (.) D) V over each whole sequence, D[n, m] =
 * g^(n-m) for n >= m, else 0 ("Summary": the parallel form is the training
 * form). `g` NULL: o receives the raw retention output. Workspace: at least
 * retention_parallel_workspace_bytes(desc) bytes (0 when there is no
 * rotation; then `workspace` may be NULL). */
size_t retention_parallel_workspace_bytes(const ret_desc_t *desc);
ret_status_t retention_parallel_fwd(const ret_desc_t *desc, const void *q, const void *k, const void *v,
                                    const void *g, void *o, void *workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* Chunkwise recurrent form ("Summary": parallel inside a chunk, the recurrent
 * state passed between chunks). For chunk i of length b (the last may be
 * shorter than `chunk`):
 *     O_i = (Q_i K_i^T (.) D) V_i + (Q_i R_{i-1}) (.) xi,   xi_r = g^(r+1)
 *     R_i = K_i^T (V_i (.) zeta) + g^b R_{i-1},            zeta_r = g^(b-1-r)
 * R_{-1} = state_in (NULL: zeros). state_out (NULL: not written) receives the
 * state after the last token; state_out == state_in is allowed. chunk >= 1.
 * Workspace: at least retention_chunkwise_workspace_bytes(desc, chunk) bytes,
 * never NULL (it holds the per-chunk states and the hand-off between the
 * workgroups that carry the state from chunk to chunk). Its first two int32
 * words form a control block that the call resets: after the call has
 * completed, word 0 counts the workgroups that ran and word 1 is nonzero only
 * on an error, after which the output is not valid: bit 0 (value 1) when a
 * cross-workgroup wait gave up after its bound (an internal error), bit 1
 * (value 2) for invalid packed-sequence bounds (retention_chunkwise_varlen_fwd).
 * retention_chunkwise_error reads the word. */
size_t retention_chunkwise_workspace_bytes(const ret_desc_t *desc, int32_t chunk);
ret_status_t retention_chunkwise_fwd(const ret_desc_t *desc, int32_t chunk, const void *q, const void *k,
                                     const void *v, const void *g, void *o, const float *state_in,
                                     float *state_out, void *workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* The chunkwise call of "Summary" (above), for measuring the chunkwise kernel
 * on its own against the chunkwise cost that "Key points" (fifth item) gives,
 * O(dn(b+h)): when non-NULL,
 * `before` and `after` (events created by the caller, for instance with
 * hipEventCreate) are recorded on `stream` immediately before and after the
 * launch of the chunkwise kernel, after the control-block reset and any
 * rotation pass. The events stay owned by the caller; everything else is as
 * retention_chunkwise_fwd, which equals this call with two NULL events. */
ret_status_t retention_chunkwise_fwd_timed(const ret_desc_t *desc, int32_t chunk, const void *q, const void *k,
                                           const void *v, const void *g, void *o, const float *state_in,
                                           float *state_out, void *workspace, size_t workspace_bytes,
                                           hipStream_t stream, hipEvent_t before, hipEvent_t after);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * chunkwise call above without a workspace argument. Its scratch (control
 * block, rotation, state chain, per-chunk states: the bytes
 * retention_chunkwise_workspace_bytes gives) lives in a static device array
 * of 128 MiB that the library holds on each device it runs on until the
 * process ends; a call that needs more returns RET_ERR_SCRATCH. The call
 * allocates nothing: no hipMalloc, hipFree or allocating library routine.
 * Its first call on a device looks up the array's address there. Every call
 * on one device shares that device's array and leaves its contents behind
 * (each call resets what must start at zero), so calls that overlap in time
 * on one device, on any streams, race and give wrong results: serialize
 * them. `error_word` (DEVICE int32, 4-byte aligned, may be NULL) receives
 * control word 1 of the call (0: no error; see retention_chunkwise_fwd) in
 * stream order. Arguments and errors otherwise as retention_chunkwise_fwd. */
ret_status_t retention_chunkwise_fwd_noalloc(const ret_desc_t *desc, int32_t chunk, const void *q, const void *k,
                                             const void *v, const void *g, void *o, const float *state_in,
                                             float *state_out, int32_t *error_word, hipStream_t stream);

/* Chunkwise form over packed sequences of different lengths (prefill of a
 * ragged batch; "Summary": the chunkwise form for long inputs, and the
 * serving claim that latency hardly depends on batch size or input length).
 * Every sequence is its own chunkwise recurrence, exactly as
 * retention_chunkwise_fwd computes it for that sequence alone, with its own
 * state_in/state_out slot and rotation positions pos_offset + n (n = 0 at
 * its first token).
 *     q, k          [total_tokens, heads, dk]  packed: sequence b occupies
 *     v, g, o       [total_tokens, heads, dv]  rows cu_seqlens[b] ..
 *                                               cu_seqlens[b+1]-1
 *     cu_seqlens    DEVICE int32 [batch + 1], non-decreasing, from 0 to
 *                   total_tokens (4-byte aligned)
 *     state_in/out  [batch, heads, dk, dv] fp32, as retention_chunkwise_fwd
 * desc->batch is the number of sequences and desc->seqlen an upper bound on
 * every length (it sizes the launch and the workspace; the rotation table
 * covers that many positions). 0 <= total_tokens <= batch * seqlen; empty
 * sequences are allowed (their state_out = state_in, or zeros). Rows of `o`
 * outside every sequence are not written. The host cannot read cu_seqlens:
 * the kernels clamp each sequence's rows into [0, total_tokens) and its
 * length to seqlen, so no access leaves the tensors whatever it holds, and a
 * clamp sets bit 1 (value 2) of control word 1 (see retention_chunkwise_fwd;
 * the output is then not valid). Workspace: at least
 * retention_chunkwise_varlen_workspace_bytes(desc, chunk) bytes, never NULL:
 * the chunkwise call's workspace plus a schedule of the launch (16 bytes per
 * workgroup), so that the workgroups of chunks past a sequence's end come
 * last and leave at once. */
size_t retention_chunkwise_varlen_workspace_bytes(const ret_desc_t *desc, int32_t chunk);
ret_status_t retention_chunkwise_varlen_fwd(const ret_desc_t *desc, int32_t chunk, const int32_t *cu_seqlens,
                                            int64_t total_tokens, const void *q, const void *k, const void *v,
                                            const void *g, void *o, const float *state_in, float *state_out,
                                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Recurrent form, one decode step for a batch of single tokens (desc->seqlen
 * must be 1): state <- g * state + k^T v, then o = q state ("Summary": O(1)
 * per token, no KV cache). `state` is read and written in place. The rotation
 * uses position desc->pos_offset for every sequence of the batch. */
ret_status_t retention_recurrent_step(const ret_desc_t *desc, const void *q, const void *k, const void *v,
                                      const void *g, void *o, float *state, hipStream_t stream);

/* The same step with one rotation position per sequence, for serving a
 * batch whose sequences sit at different lengths ("Key points", first item:
 * decode latency stays nearly flat as the batch or the input grows; "Summary":
 * the positions are encoded like xPos, i.e. by each token's own position):
 * `positions` is a
 * DEVICE array of `batch` int64 positions, 8-byte aligned, each in
 * [0, 2^52] or negative (not checked: it lives on the device), read by the
 * step's kernel in place of desc->pos_offset. A negative position marks an
 * inactive slot of the batch: its state is left as it is and its output row
 * is zero. Without rotation the positions only mark the inactive slots. */
ret_status_t retention_recurrent_step_positions(const ret_desc_t *desc, const void *q, const void *k,
                                                const void *v, const void *g, void *o, float *state,
                                                const int64_t *positions, hipStream_t stream);

/* Backward of the parallel form: the gradients of sum(dout (.) out), with
 * out the output of retention_parallel_fwd on the same (desc, q, k, v, g),
 * with respect to q, k, v and (when g != NULL) g. All of q, k, v, g, dout,
 * dq, dk, dv and dg share the layout and dtype of the forward's tensors; dg
 * must be NULL exactly when g is. The outputs must not overlap each other,
 * the inputs or the workspace.
 *
 * Computed as the chain rule of the forward's definition (the parallel form
 * is the training form, "Summary"): through the swish gate and GroupNorm
 * (the raw retention output is recomputed), then, with A = (Q' K'^T) (.) D,
 *     dV = A^T dO,   dQ' = ((dO V^T) (.) D) K',   dK' = ((dO V^T) (.) D)^T Q',
 * each a causal retention product (the last two on token-reversed
 * sequences), and dq, dk turned back by the rotation's angles. Gradients are
 * stored in the input dtype; products accumulate in fp32.
 *
 * Workspace: at least retention_parallel_bwd_workspace_bytes(desc, g != NULL)
 * bytes (0 without rotation and gate: workspace may then be NULL). */
size_t retention_parallel_bwd_workspace_bytes(const ret_desc_t *desc, int32_t has_gate);
ret_status_t retention_parallel_bwd(const ret_desc_t *desc, const void *q, const void *k, const void *v,
                                    const void *g, const void *dout, void *dq, void *dk, void *dv, void *dg,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Backward of the chunkwise form (no carried state: state_in and state_out
 * of the forward both NULL): the same gradients as retention_parallel_bwd,
 * since the two forms compute one function ("Summary": the forms are
 * equivalent), with each product run as the chunkwise form at `chunk`, so the
 * cost grows linearly with the sequence. Arguments as retention_parallel_bwd,
 * plus chunk >= 1. Workspace: at least
 * retention_chunkwise_bwd_workspace_bytes(desc, chunk, g != NULL) bytes; its
 * first bytes are the chunkwise call's control block. */
size_t retention_chunkwise_bwd_workspace_bytes(const ret_desc_t *desc, int32_t chunk, int32_t has_gate);
ret_status_t retention_chunkwise_bwd(const ret_desc_t *desc, int32_t chunk, const void *q, const void *k,
                                     const void *v, const void *g, const void *dout, void *dq, void *dk, void *dv,
                                     void *dg, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* The chunkwise backward with a carried state: the forward ran from
 * `state_in` (DEVICE fp32 [batch, heads, dk, dv]) and the loss may also
 * depend on its state_out, whose gradient `d_state_out` (same layout; NULL:
 * none) the caller passes. Besides dq, dk, dv, dg it writes `d_state_in`, the
 * gradient with respect to state_in (non-NULL exactly when state_in is). The
 * state terms run through the same three products: S0^T as the dq
 * product's initial state, dS_out / g (per head) as the reversed products'
 * initial states, and d_state_in = g Z^T from the reversed dk product's
 * final state Z. Every decay must be >= 2^-60 when d_state_out is given
 * (RET_ERR_GAMMA otherwise). Workspace: at least
 * retention_chunkwise_bwd_state_workspace_bytes(desc, chunk, g != NULL). */
size_t retention_chunkwise_bwd_state_workspace_bytes(const ret_desc_t *desc, int32_t chunk, int32_t has_gate);
ret_status_t retention_chunkwise_bwd_state(const ret_desc_t *desc, int32_t chunk, const void *q, const void *k,
                                           const void *v, const void *g, const void *dout, const float *state_in,
                                           const float *d_state_out, void *dq, void *dk, void *dv, void *dg,
                                           float *d_state_in, void *workspace, size_t workspace_bytes,
                                           hipStream_t stream);

/* Retention score map of one query token over the tokens before it: the
 * magnitude of each head's query-key dot product, weighted by that head's
 * decay of the distance (the parallel form's weights), summed across heads
 * ("Visualization of the retention mechanism", SpiralAI model card page):
 *     scores[b, m] = sum_h g_h^(n-m) |q'_{b,n,h} . k'_{b,m,h}|   (m <= n)
 * and 0 for m > n, with q', k' rotated by position and n = `query`
 * (-1: the last token). scores: DEVICE fp32 [batch, seqlen], 16-byte
 * aligned. Workspace: retention_score_map_workspace_bytes(desc) bytes (0
 * without rotation; then `workspace` may be NULL). */
size_t retention_score_map_workspace_bytes(const ret_desc_t *desc);
ret_status_t retention_score_map(const ret_desc_t *desc, const void *q, const void *k, int32_t query, float *scores,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Control word 1 of a chunkwise workspace, after the call that used it:
 * waits for the work enqueued on `stream` (hipStreamSynchronize), then copies
 * the word to *error_word (HOST pointer). The chunkwise calls
 * (retention_chunkwise_fwd, _fwd_timed, _varlen_fwd, _bwd, _bwd_state) reset
 * it at their start and set it only on an error, after which their outputs
 * are not valid: bit 0 (value 1) when a wait between the workgroups that
 * carry the state from chunk to chunk gave up after its bound, bit 1 (value
 * 2) for packed-sequence bounds that had to be clamped. The backward's
 * word covers all of its launches. The chunkwise form itself is the one of
 * "Summary": the recurrent state passed between chunks. Returns RET_ERR_NULL,
 * RET_ERR_WORKSPACE (fewer than 8 bytes), RET_ERR_ALIGN or RET_ERR_HIP (the
 * copy or the wait failed, for instance after a fault of an earlier kernel). */
ret_status_t retention_chunkwise_error(const void *workspace, size_t workspace_bytes, int32_t *error_word,
                                       hipStream_t stream);

/* Human-readable name of a status code (static string, never NULL). */
const char *retention_status_string(ret_status_t status);

/* Version of this ABI (incremented on incompatible change). */
int32_t retention_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RETENTION_H */

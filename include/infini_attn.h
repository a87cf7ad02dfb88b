/*
 * infini_attn.h -- C ABI of the Infini-attention segment forward for AMD MI355X (gfx950).
 *
 * The method: "Leave No Context Behind: Efficient Infinite Context Transformers
 * with Infini-attention" (Munkhdalai, Faruqui, Golovnev; arXiv 2404.07143), as
 * restated on the pages "精读笔记：Infini-attention" (sections 3.1-3.8),
 * "忘记遗忘：解锁无限上下文的 Infini-attention" (section 2) and
 * "第24章 Sparse与Infinite Attention" (sections 24.4-24.5).
 *
 * For every (batch b, head h) the sequence is cut into segments of N tokens and
 * the segments are processed in order.  Segment s of head (b, h) computes
 *
 *   A_dot = softmax(scale * Q K^T, causal inside the segment) V        (section 3.1)
 *   A_mem = sigma(Q) M_{s-1} / (sigma(Q) z_{s-1}),  sigma = ELU + 1      (section 3.3)
 *   A     = g * A_mem + (1 - g) * A_dot,  g = sigmoid(beta_h)           (section 3.5)
 *
 * and then updates the compressive state (section 3.4):
 *
 *   linear: M_s = M_{s-1} + sigma(K)^T V
 *   delta : M_s = M_{s-1} + sigma(K)^T (V - sigma(K) M_{s-1} / (sigma(K) z_{s-1}))
 *   both  : z_s = z_{s-1} + sum_t sigma(K_t)
 *
 * Conventions fixed by this library: M_0 = 0, z_0 = 0; in the first segment after
 * init or reset A_mem = 0 and the delta correction is 0 (so the first delta
 * update equals the linear one).  "First" is decided by the state's segment
 * counter.  scale <= 0 selects 1/sqrt(d_key).  The delta correction is
 * segment-batched: every token of segment s reads M_{s-1}, z_{s-1}.
 *
 * Memory and layouts.  Every tensor pointer is a DEVICE pointer to contiguous
 * row-major memory owned by the caller; the library never allocates, frees or
 * keeps device memory and holds no global state besides a thread-local error
 * string.
 *   q, k  : [B, H, L, d_key]   dtype of the state (fp32 or bf16)
 *   v, out: [B, H, L, d_value] same dtype
 *   beta  : [H] fp32, one gate logit per head shared over the batch (section 3.5)
 *   M     : [B, H, d_key, d_value] fp32;  z: [B, H, d_key] fp32
 * out must not alias q, k, v, M, z or the workspace.
 *
 * Supported shapes.  bf16 with d_key == d_value in {64, 128} and N a positive
 * multiple of 64 runs the MFMA kernels (any N of that form).  Every other state
 * with 1 <= d_key, d_value <= 128 and 1 <= N <= 4096 (fp32, and bf16 with other
 * widths, d_key != d_value or a ragged N) runs the VALU kernels, one segment per
 * launch, with the same arithmetic in fp32.  Other shapes return
 * INFINI_EUNSUPPORTED.  The layer and kernel-linear-attention entry points run
 * the MFMA shapes only.
 *
 * Accuracy.  sigma(q) and sigma(K) enter the bf16 kernels' memory products as
 * (sigma - 1) or as an exact pair of bf16 parts, so keys and queries near 0
 * (sigma ~ 1) keep their full precision; the retrieval of the fused kernel forms
 * sigma(q) M as colsum(M) + (sigma(q) - 1) M, which loses relative precision for
 * queries far below 0 (sigma(q) << 1, about 1e-2 relative at q ~ -4).
 *
 * Errors.  Every entry point validates all of its arguments before making any
 * HIP call; on an error it enqueues nothing, leaves *st unchanged and returns a
 * negative infini_status; infini_attn_last_error() then describes the problem.
 * Work is enqueued on `stream` (a hipStream_t; NULL is the null stream) and the
 * call returns without synchronising; a launch failure returns INFINI_EHIP and a
 * device fault surfaces at the caller's next synchronisation.
 *
 * Threads.  One state must not be used from two threads or two streams at once.
 * The counter segments_done advances on the host at enqueue time.
 *
 * Entry points beyond the segment stream (each documented at its declaration):
 * the open segment (tokens in any number per call, single-token decode, ragged
 * tails: infini_attn_open_segment_init / _append_workspace_bytes / _append), the
 * gradients of a forward_sequence call (infini_attn_backward_sequence), the
 * layer with its Q/K/V and output projections (infini_attn_layer_forward) and
 * causal kernel linear attention on the same state (infini_attn_kernel_linear_attention).
 */
#ifndef INFINI_ATTN_H
#define INFINI_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  INFINI_OK = 0,
  INFINI_EINVAL = -1,        /* a null pointer, a non-positive or inconsistent size */
  INFINI_EUNSUPPORTED = -2,  /* a valid shape or dtype this build has no kernel for */
  INFINI_EWORKSPACE = -3,    /* workspace missing or smaller than infini_attn_workspace_bytes */
  INFINI_EHIP = -4           /* a HIP runtime call or kernel launch failed */
} infini_status;

typedef enum { INFINI_RULE_LINEAR = 0, INFINI_RULE_DELTA = 1 } infini_rule;
typedef enum { INFINI_F32 = 0, INFINI_BF16 = 1 } infini_dtype;

/* Caller-allocated plain struct.  Fill it only through infini_attn_init_state. */
typedef struct {
  int32_t batch, heads, d_key, d_value, segment_len; /* B, H, d_key, d_value, N */
  int32_t dtype;          /* infini_dtype of q, k, v and out */
  int32_t rule;           /* infini_rule */
  float scale;            /* softmax scale actually used (1/sqrt(d_key) if given <= 0) */
  float *M;               /* device fp32 [B, H, d_key, d_value], caller-owned */
  float *z;               /* device fp32 [B, H, d_key], caller-owned */
  int64_t segments_done;  /* segments folded into (M, z); 0 => next segment reads an empty memory */
} infini_attn_state;

/* Validates the configuration, fills *st, zeroes M and z on `stream` and sets the
 * counter to 0 (the state of a fresh stream: M_0 = 0, z_0 = 0).  The state is the
 * compressive memory of section 3.4 of "精读笔记：Infini-attention", one M
 * (d_key x d_value) and one z (d_key) per head (section 3.6), d_key (d_value + 1)
 * values per head (section 3.7, Table 1).  M and z: device fp32, 4-byte aligned,
 * caller-owned, not overlapping.  Errors: EINVAL for a NULL pointer, a
 * non-positive size, an unknown dtype or rule, an infinite scale; EUNSUPPORTED
 * for the shapes listed above. */
int infini_attn_init_state(infini_attn_state *st, int32_t batch, int32_t heads,
                           int32_t d_key, int32_t d_value, int32_t segment_len,
                           int32_t dtype, int32_t rule, float scale,
                           float *M, float *z, void *stream);

/* Bytes of device workspace that forward_sequence needs for seq_len tokens
 * (forward_segment: seq_len = segment_len).  Returns 0 for an invalid state or a
 * seq_len that is not a positive multiple of the segment length. */
size_t infini_attn_workspace_bytes(const infini_attn_state *st, int64_t seq_len);

/* Processes the S = seq_len / N segments of every (b, h) in order, starting from
 * the state's (M, z, segments_done), writes A to out and leaves (M_S, z_S) in the
 * state; segments_done += S.  Each segment is the forward of section 3.8 of
 * "精读笔记：Infini-attention" (steps 1-5): local causal attention (section 3.1),
 * retrieval (section 3.3), gate (section 3.5), memory update (section 3.4, the
 * delta fraction as written in section 2.1 of "忘记遗忘：解锁无限上下文的
 * Infini-attention"); the order retrieve-then-update follows section 24.5 of
 * "第24章 Sparse与Infinite Attention".  q, k, v, out hold seq_len tokens per
 * (b, h), 16-byte aligned for bf16 and 4-byte for fp32.  beta: device fp32 [H].
 * workspace: device memory of at least infini_attn_workspace_bytes(st, seq_len)
 * bytes, 256-byte aligned, contents irrelevant on entry and undefined on return.
 * Errors: EINVAL (NULL pointers, seq_len not a positive multiple of N,
 * misalignment, out aliasing an input or the state), EWORKSPACE (workspace
 * missing, too small, misaligned or aliasing), EUNSUPPORTED (a launch grid above
 * 2^31 workgroups: split the call), EHIP (a launch failed).
 * On the bf16 delta path a long stream with few heads runs its sequential memory
 * chain on a side stream of the library's (one per device, default priority,
 * created on the first such call and kept until the process ends) beside the
 * attention on `stream`; the call's work is still ordered on `stream` (it waits
 * for the side stream before its last kernel) and the results are the same. */
int infini_attn_forward_sequence(infini_attn_state *st, const void *q, const void *k,
                                 const void *v, int64_t seq_len, const float *beta,
                                 void *out, void *workspace, size_t workspace_bytes,
                                 void *stream);

/* forward_sequence for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): no
 * workspace argument; the call uses a scratch array of
 * infini_attn_noalloc_scratch_bytes() bytes (64 MiB) that the library keeps in
 * device memory, one per GPU, for the life of the process, and calls no
 * allocating routine.  Calls whose workspace (infini_attn_workspace_bytes) exceeds
 * it return INFINI_EWORKSPACE without enqueueing anything: split the stream into
 * shorter calls.  Every call on a GPU shares that GPU's array (its contents on
 * entry do not matter), so calls that overlap on one GPU (other streams, other
 * threads) race: serialise them.  Otherwise as forward_sequence, bitwise the same
 * results. */
int infini_attn_forward_sequence_noalloc(infini_attn_state *st, const void *q, const void *k,
                                         const void *v, int64_t seq_len, const float *beta,
                                         void *out, void *stream);
/* Size of the scratch array of infini_attn_forward_sequence_noalloc. */
size_t infini_attn_noalloc_scratch_bytes(void);

/* forward_sequence that also records caller-created HIP events (hipEvent_t, as
 * void*) on `stream` at the stage boundaries, for profiling tools:
 *   events[0] before the first kernel, events[1] after the memory-state stage
 *   (linear contributions + prefix scan, or the delta chain; for fp32 after the
 *   last segment's update), events[2] after the fused attention stage.
 * n_events must be 3 and every event non-NULL; otherwise INFINI_EINVAL.  The
 * arithmetic and results are those of forward_sequence. */
int infini_attn_forward_sequence_profiled(infini_attn_state *st, const void *q, const void *k,
                                          const void *v, int64_t seq_len, const float *beta,
                                          void *out, void *workspace, size_t workspace_bytes,
                                          void *stream, void *const *events, int32_t n_events);

/* One segment: the same as forward_sequence with seq_len = segment_len (the
 * per-segment recurrence of section 3.4 of "精读笔记：Infini-attention": the
 * state carries M_{s-1}, z_{s-1} from one call to the next).  A stream fed
 * segment by segment gives bitwise the same results as one forward_sequence
 * call over the whole stream, except at d_key = 128 when that call holds at least
 * as many (b, h, segment) tiles as the device has compute units: its per-segment
 * sums sigma(K)^T V and sum sigma(K) are then formed in another order, and the
 * results agree up to that fp32 rounding.  Arguments and errors as
 * forward_sequence. */
int infini_attn_forward_segment(infini_attn_state *st, const void *q, const void *k,
                                const void *v, const float *beta, void *out,
                                void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Open segment: streaming inference and ragged tails ("streaming inference",
 * abstract of the page "精读笔记：Infini-attention"; point 4 of the key-idea list
 * of the page "忘记遗忘：解锁无限上下文的 Infini-attention").
 *
 * Tokens may arrive in any number per call, one at a time (decode) included.  A
 * token that arrives before its segment is complete is answered with the
 * segment as it stands: local causal attention over the segment's tokens that
 * have arrived (itself included), retrieval from (M, z) as of the segment's
 * start, the gate.  The segment is folded into (M, z) when its N-th token
 * arrives.  Because the local attention is causal, every token gets the output
 * it gets when its segment is processed whole; appending whole segments at a
 * segment boundary runs the segment path of forward_sequence (bitwise the same
 * results).  The keys and values of the open segment live in caller-owned
 * device buffers; the fill level is kept on the host. */
typedef struct {
  void *k_open;    /* device [B, H, N, d_key], dtype of the state, caller-owned */
  void *v_open;    /* device [B, H, N, d_value], caller-owned */
  int32_t filled;  /* tokens of the open segment held in k_open / v_open, 0 <= filled < N */
} infini_attn_open_segment;

/* Binds the buffers to *os and empties the open segment (filled = 0); no HIP
 * call.  The buffers must not overlap each other or the state.  Call it again
 * after infini_attn_reset. */
int infini_attn_open_segment_init(const infini_attn_state *st, infini_attn_open_segment *os,
                                  void *k_open, void *v_open);

/* Bytes of device workspace that infini_attn_append needs for n_tokens tokens
 * (0 for an invalid state or n_tokens < 1). */
size_t infini_attn_append_workspace_bytes(const infini_attn_state *st, int64_t n_tokens);

/* Appends n_tokens tokens per (b, h) to the stream of *st / *os and writes their
 * outputs: q, k: [B, H, n_tokens, d_key]; v, out: [B, H, n_tokens, d_value];
 * beta: device fp32 [H].  Completed segments are folded into (M, z)
 * (segments_done += 1 each) and the open segment restarts empty; os->filled
 * ends at (filled + n_tokens) % N.  The workspace rules are those of
 * forward_sequence with infini_attn_append_workspace_bytes.  out must not alias
 * q, k, v, the state, the open-segment buffers or the workspace.  Do not mix
 * with forward_sequence / forward_segment while the open segment holds tokens
 * (those start at a segment boundary). */
int infini_attn_append(infini_attn_state *st, infini_attn_open_segment *os, const void *q,
                       const void *k, const void *v, int64_t n_tokens, const float *beta,
                       void *out, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Gradients (training through the layer: section 4 of the page
 * "精读笔记：Infini-attention"; the pages give the forward equations of sections
 * 3.1, 3.3, 3.4 and 3.5, and these are their derivatives).
 *
 * For a forward_sequence call that started from the state *st (M, z and
 * segments_done as they were BEFORE that call: keep a copy, the forward updates
 * them in place) over q, k, v, beta, and the loss
 *     <dout, A> + <dM, M_S> + <dz, z_S>
 * (A the forward's output, M_S, z_S the state after it), writes dq, dk, dv (the
 * dtype of the state, layouts of q, k, v), dbeta (fp32 [H], summed over the
 * batch), and, when non-NULL, dM0, dz0 (fp32, layouts of M and z: the gradient
 * of the state the call started from, to chain calls backwards).  dM and dz
 * (fp32, the gradient of the final state) may be NULL for zero.  *st is not
 * changed.  The forward is recomputed from the inputs (nothing has to be kept
 * from it besides the starting state).  No output may overlap another, the
 * workspace, the inputs or the state.  Errors as for forward_sequence. */
size_t infini_attn_backward_workspace_bytes(const infini_attn_state *st, int64_t seq_len);
int infini_attn_backward_sequence(const infini_attn_state *st, const void *q, const void *k,
                                  const void *v, int64_t seq_len, const float *beta,
                                  const void *dout, const float *dM, const float *dz, void *dq,
                                  void *dk, void *dv, float *dbeta, float *dM0, float *dz0,
                                  void *workspace, size_t workspace_bytes, void *stream);

/* Training pair: a forward that keeps the local attention's softmax statistics,
 * and a backward that uses them with the forward's output instead of
 * recomputing the first of its two sweeps over the keys (the same derivatives
 * as infini_attn_backward_sequence; section 3.1 of the page "精读笔记：
 * Infini-attention" for the causal softmax, 3.3-3.5 for the memory and gate).
 * bf16 MFMA path only (d_key = d_value in {64, 128}, segment_len a multiple of
 * 64): INFINI_EUNSUPPORTED otherwise.
 *
 * forward_sequence_train: forward_sequence (the same arguments, the same out and
 * state, bitwise) that also writes lse, fp32 [B, H, seq_len] (4-byte aligned,
 * caller-owned, overlapping nothing else): per query row t, log2 of
 * sum over the causal keys j <= t of 2^(scale q_t.k_j log2 e), i.e. the
 * row's softmax log-normaliser in base 2 of the scores scale q.k log2 e.
 *
 * backward_sequence_saved: backward_sequence given out (the forward's output A,
 * bf16 [B, H, seq_len, d_value], 16-byte aligned) and lse from a
 * forward_sequence_train call over the same inputs and starting state; both are
 * read only and may not overlap an output or the workspace.  Workspace size
 * from infini_attn_backward_workspace_bytes.  Other arguments, results and
 * errors as backward_sequence. */
int infini_attn_forward_sequence_train(infini_attn_state *st, const void *q, const void *k,
                                       const void *v, int64_t seq_len, const float *beta, void *out,
                                       float *lse, void *workspace, size_t workspace_bytes,
                                       void *stream);
int infini_attn_backward_sequence_saved(const infini_attn_state *st, const void *q, const void *k,
                                        const void *v, int64_t seq_len, const float *beta,
                                        const void *out, const float *lse, const void *dout,
                                        const float *dM, const float *dz, void *dq, void *dk, void *dv,
                                        float *dbeta, float *dM0, float *dz0, void *workspace,
                                        size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * The layer: the projections on either side of the segment stream
 * (section 3.1 of the page "精读笔记：Infini-attention": Q = X W_Q, K = X W_K,
 * V = X W_V per head; section 3.6: O = [A^1; ...; A^H] W_O).  bf16 path only.
 *
 * x, y: [B, seq_len, d_model] bf16; w_qkv: [d_model, H (2 d_key + d_value)] bf16,
 * its columns the H query heads (d_key each, head h at h d_key), then the H key
 * heads, then the H value heads; w_o: [H d_value, d_model] bf16, its rows the
 * heads' outputs in head order.  Runs y = concat_h(A_h) w_o with A_h the stream
 * of head h over the projected q, k, v (forward_sequence semantics: the state
 * advances by seq_len / segment_len segments).  d_model a multiple of 64;
 * x, the weights and y 16-byte aligned; y must not alias the inputs, the state
 * or the workspace.  The workspace holds the projected q, k, v, the heads'
 * outputs and the forward's workspace.  Errors as for forward_sequence;
 * INFINI_EUNSUPPORTED for the fp32 path. */
size_t infini_attn_layer_workspace_bytes(const infini_attn_state *st, int32_t d_model, int64_t seq_len);
int infini_attn_layer_forward(infini_attn_state *st, const void *x, int32_t d_model, const void *w_qkv,
                              const void *w_o, int64_t seq_len, const float *beta, void *y,
                              void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Causal kernel linear attention (section 24.4 of the page "第24章 Sparse与
 * Infinite Attention"): out_i = phi(q_i)^T S_i / (phi(q_i)^T Z_i) with the
 * prefix states S_i = M_0 + sum_{j <= i} phi(k_j) v_j^T and Z_i = z_0 +
 * sum_{j <= i} phi(k_j) over the stream (phi = ELU + 1; the query's own key
 * included).  The state carries (S, Z) across calls exactly as the linear rule
 * carries (M, z): it must use INFINI_RULE_LINEAR, and its segment length is the
 * chunk the kernels work in (any multiple of 64; the result does not depend on
 * it beyond rounding).  q, k, v, out [B, H, seq_len, d] bf16, 16-byte aligned;
 * seq_len a multiple of segment_len; the workspace of forward_sequence
 * (infini_attn_workspace_bytes).  M, z end as S, Z of the last token and
 * segments_done advances by seq_len / segment_len.  bf16 path only. */
int infini_attn_kernel_linear_attention(infini_attn_state *st, const void *q, const void *k,
                                        const void *v, int64_t seq_len, void *out, void *workspace,
                                        size_t workspace_bytes, void *stream);

/* M, z <- 0 on `stream`; segments_done <- 0: the empty memory M_0 = 0, z_0 = 0 a
 * stream starts from (the first segment then reads A_mem = 0, the convention of
 * this library for section 3.3's 0 / 0 of "精读笔记：Infini-attention").  No
 * allocation; EINVAL for an invalid state. */
int infini_attn_reset(infini_attn_state *st, void *stream);

/* Message of the last failed call on this thread ("" if none). */
const char *infini_attn_last_error(void);

/* Library ABI version, currently 1. */
int infini_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* INFINI_ATTN_H */

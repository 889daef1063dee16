/*
 * gdr.h — gated delta-rule matrix-memory kernels for AMD MI355X (gfx950).
 *
 * C ABI of libgdr.so. Every entry point takes plain device pointers, sizes and
 * a HIP stream, validates its arguments on the host, enqueues its kernels on
 * that stream and returns without synchronising. No entry point allocates or
 * frees memory, and the library keeps no hidden state between calls: the
 * caller owns every buffer (the one exception is gdr_chunk_fwd_noalloc, whose
 * records go through a static per-device scratch array, see there). Calls are
 * reentrant; calls that write the same buffers must be ordered by the caller
 * (same stream or events).
 *
 * Notation follows "Muir: Linear Attention with Sensitivity-Allocated Gating
 * and Matched-Filter Readout" (§2.1 eq.(1)): row vectors, state S[d_k, d_v]
 * acted on from the left, readout o = q S.
 *
 * Layouts: all tensors are contiguous, last dimension fastest.
 *   sequence tensors  [B, H, T, d]     (head-major: one head's tokens are contiguous)
 *   states            [B, H, d_k, d_v] (float32, d_v fastest)
 *   decode tensors    [N, H, d]
 *
 * Supported sizes: d_k, d_v in {16, 32, 64, 128} for the gated delta rule,
 * {16, 32, 64, 128, 256} for mLSTM; chunk in {16, 32, 64}; any T >= 1 (a
 * ragged last chunk behaves as if padded with identity steps alpha = 1, k = 0,
 * v = 0, whose outputs are discarded). For gdr_chunk_fwd with float32 inputs
 * and d_k >= 64 the chunk must be at most 32 (fp32 operands take twice the
 * LDS); gdr_chunk_fwd_ws has no such limit.
 * Alignment: every pointer must be 16-byte aligned.
 *
 * Preconditions not checked on the hot path: alpha (and RWKV-7's w) in
 * (0, 1]; inputs finite; output buffers do not overlap input buffers except
 * where stated. The overlap rule is checked on the host in every build. The
 * value rules are checked only by the debug library, libgdr_debug.so (the
 * same sources built with GDR_DEBUG defined; the Python binding loads it when
 * the environment variable GDR_DEBUG is set to 1): before enqueuing any compute
 * kernel each entry point reads its inputs once on the GPU, waits for the
 * result and returns GDR_ERR_PRECONDITION, with nothing enqueued, when an
 * element breaks its rule; gdr_debug_violation then names the arguments.
 * Those checks synchronise the stream, so the debug library's entry points
 * cannot be captured into a HIP graph.
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. Negative values are errors; no kernel was enqueued. */
#define GDR_OK               0
#define GDR_ERR_NULL        -1  /* a required pointer is NULL */
#define GDR_ERR_SHAPE       -2  /* a size is out of range (e.g. T < 1, B < 1) */
#define GDR_ERR_DTYPE       -3  /* unknown dtype code */
#define GDR_ERR_UNSUPPORTED -4  /* sizes valid but not built (d or chunk outside the supported set) */
#define GDR_ERR_ALIGN       -5  /* a pointer is not 16-byte aligned */
#define GDR_ERR_LAUNCH      -6  /* the HIP runtime rejected a kernel launch */
#define GDR_ERR_ALIAS       -7  /* an output buffer overlaps an input buffer */
#define GDR_ERR_WORKSPACE   -8  /* workspace smaller than gdr_chunk_workspace_size reports */
#define GDR_ERR_TOO_LARGE   -9  /* one head needs more than gdr_chunk_fwd_noalloc's static scratch */
#define GDR_ERR_PRECONDITION -10 /* debug library only: a non-finite input, or a decay outside (0, 1] */

/* Input/output element types. States (S, C, n, m) are always float32. */
#define GDR_F32  0
#define GDR_BF16 1

/*
 * gdr_chunk_fwd — chunkwise-parallel forward of the channel-wise gated delta
 * rule over whole sequences.
 *
 * Computes, for every (b, h) and t = 1..T, the recurrence of "Muir: ...",
 * §2.1 eq.(1):
 *     S_t = (I - k_t^T (b_t * k_t)) Diag(alpha_t) S_{t-1} + k_t^T (w_t * v_t),
 *     o_t = q_t S_t,
 * starting from S_0, and returns all o_t and S_T. It evaluates the recurrence
 * chunk by chunk with the UT form of §2.2 (T V~ = V^ - K^_pi S_0, O = Q_pi S_0
 * + M V~, S_C = Diag(pi_C) S_0 + K~^T V~), keeping every decay factor a
 * product of alphas over an interval so that nothing divides by a vanishing
 * cumulative decay.
 *
 *   q, k, alpha, b  [B,H,T,dk]  input dtype (query, key, decay gate, erase gate)
 *   v, w            [B,H,T,dv]  input dtype (value, write gate)
 *   S0              [B,H,dk,dv] float32 initial state, or NULL for zeros
 *   o               [B,H,T,dv]  output, input dtype
 *   S_out           [B,H,dk,dv] float32 final state, or NULL to skip; may
 *                   equal S0 (in-place update), must not otherwise overlap it
 *   chunk           chunk length C (16, 32 or 64; with float32 inputs and
 *                   d_k >= 64 at most 32 here, as fp32 operands take twice
 *                   the LDS: C = 64 then returns GDR_ERR_UNSUPPORTED, while
 *                   gdr_chunk_fwd_ws takes it)
 *   dtype           GDR_F32 or GDR_BF16 (applies to q, k, v, alpha, b, w, o)
 *   stream          hipStream_t to enqueue on (NULL = default stream)
 * Returns GDR_OK or a negative GDR_ERR_* code.
 */
int gdr_chunk_fwd(const void* q, const void* k, const void* v,
                  const void* alpha, const void* b, const void* w,
                  const float* S0, void* o, float* S_out,
                  int B, int H, int T, int dk, int dv, int chunk, int dtype,
                  void* stream);

/*
 * gdr_chunk_workspace_size — bytes of device workspace gdr_chunk_fwd_ws needs
 * for these sizes: one record per (b, h, chunk) of C*dk*3 + dv*C + C*C
 * elements of the input dtype plus dk float32 values.
 * Writes the size to *bytes (0 on error). Returns GDR_OK or a GDR_ERR_* code.
 */
int gdr_chunk_workspace_size(int B, int H, int T, int dk, int dv, int chunk,
                             int dtype, size_t* bytes);

/*
 * gdr_chunk_fwd_ws — the computation of gdr_chunk_fwd (same arguments, same
 * results up to rounding) as two kernels, which is the fast form for long
 * sequences:
 *   1. every (b, h, chunk) in parallel: the state-independent part of the
 *      chunkwise form of "Muir: ...", §2.2 with the fused right-hand side of
 *      §4.2, [U | Y] = T^{-1} [V^ | K^_pi], together with M, Q_pi, K~^T and
 *      pi_C, written to `workspace`;
 *   2. one pass over the chunks of each head: V~ = U - Y S_0,
 *      O = Q_pi S_0 + M V~, S_C = Diag(pi_C) S_0 + K~^T V~.
 *
 *   workspace        device buffer of at least gdr_chunk_workspace_size()
 *                    bytes, 16-byte aligned, owned by the caller; its contents
 *                    on entry are ignored and on return are unspecified. It
 *                    must not overlap any other argument, and calls that run
 *                    concurrently need separate workspaces.
 *   workspace_bytes  its size in bytes
 * Other arguments as for gdr_chunk_fwd. Returns GDR_OK or a negative
 * GDR_ERR_* code (GDR_ERR_WORKSPACE if the workspace is too small).
 */
int gdr_chunk_fwd_ws(const void* q, const void* k, const void* v,
                     const void* alpha, const void* b, const void* w,
                     const float* S0, void* o, float* S_out,
                     int B, int H, int T, int dk, int dv, int chunk, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdr_chunk_intra, gdr_chunk_scan — the two kernels of gdr_chunk_fwd_ws as
 * separate calls (same workspace, same stream order): gdr_chunk_intra reads
 * the inputs and fills the workspace with the state-independent part of every
 * chunk; gdr_chunk_scan then walks the chunks of every head from S0 and
 * writes o and S_out. Called in this order with the same sizes they compute
 * exactly what gdr_chunk_fwd_ws computes. Arguments and errors as for
 * gdr_chunk_fwd_ws; gdr_chunk_scan reads a workspace that gdr_chunk_intra
 * filled for the same B, H, T, dk, dv, chunk and dtype (not checked).
 */
int gdr_chunk_intra(const void* q, const void* k, const void* v,
                    const void* alpha, const void* b, const void* w,
                    int B, int H, int T, int dk, int dv, int chunk, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream);
int gdr_chunk_scan(const void* workspace, size_t workspace_bytes,
                   const float* S0, void* o, float* S_out,
                   int B, int H, int T, int dk, int dv, int chunk, int dtype,
                   void* stream);

/*
 * gdr_chunk_bwd_workspace_size, gdr_chunk_bwd — gradients of the chunkwise
 * forward ("Muir: ...", §4.2 "Custom Backward Pass"): for a scalar loss J with
 * dO = dJ/do and dS_T = dJ/dS_T, returns dJ/dq, dJ/dk, dJ/dv, dJ/dalpha,
 * dJ/db, dJ/dw and dJ/dS0 of the recurrence of §2.1 eq.(1).
 *
 * The chunk readout and state update of eq.(10) are differentiated with
 * matrix products, the triangular solve through the transposed solve
 * d[V^ | K^_pi] = T^{-T} d[U | Y] and dL = -stril(d[V^ | K^_pi] [U | Y]^T),
 * and the decay-scaled Gram products back to q, k, b and the cumulative
 * log-decay, whose reverse cumulative sum gives d log alpha (dalpha =
 * d log alpha / alpha, so alpha must be > 0 here).
 *
 *   q, k, v, alpha, b, w, S0   the forward's inputs (as gdr_chunk_fwd; S0 may
 *                              be NULL for zeros)
 *   dO        [B,H,T,dv]  input dtype, gradient of the outputs
 *   dS_T      [B,H,dk,dv] float32 gradient of the final state, or NULL (zero)
 *   dq, dk, dalpha, db  [B,H,T,dk] float32 outputs
 *   dv, dw              [B,H,T,dv] float32 outputs
 *   dS0       [B,H,dk,dv] float32 output, or NULL to skip
 *   workspace at least gdr_chunk_bwd_workspace_size bytes; it begins with
 *             the forward's records (the first gdr_chunk_workspace_size
 *             bytes of the same shapes, records only). records_ready = 1
 *             when the caller's workspace already holds them for these
 *             inputs (written by gdr_chunk_intra or gdr_chunk_fwd_ws into
 *             the same buffer), 0 to recompute them first.
 * Outputs must not overlap inputs, each other or the workspace. Returns
 * GDR_OK or a negative GDR_ERR_* code.
 */
int gdr_chunk_bwd_workspace_size(int B, int H, int T, int dk, int dv, int chunk, int dtype, size_t* bytes);
int gdr_chunk_bwd(const void* q, const void* k, const void* v,
                  const void* alpha, const void* b, const void* w,
                  const float* S0, const void* dO, const float* dS_T,
                  float* dq, float* dk_, float* dv_, float* dalpha, float* db, float* dw, float* dS0,
                  int B, int H, int T, int dk, int dv, int chunk, int dtype,
                  void* workspace, size_t workspace_bytes, int records_ready, void* stream);

/*
 * gdr_chunk_fwd_noalloc — gdr_chunk_fwd_ws without a caller workspace and
 * without any allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments, results and errors as gdr_chunk_fwd_ws minus
 * the workspace; the results equal it up to rounding, and bit for bit for
 * bfloat16 inputs with d_k, d_v and C multiples of 32 (the fragment-order
 * record, whose kernels do the same arithmetic per head whatever the batch).
 *
 * The records go through a scratch array of GDR_NOALLOC_SCRATCH_BYTES (64 MiB)
 * compiled into the library: every GPU the library runs on holds its own copy
 * from the first call on that device until the process ends. Heads are
 * processed in groups of consecutive (b, h) pairs that fit the array
 * (gdr_chunk_workspace_size(1, 1, T, ...) bytes per head; 4.75 MB at T = 4096,
 * d = 128, C = 64, so 14 heads per group), intra kernel then scan per group,
 * all on `stream`. If one head alone needs more than the array (T above about
 * 57,800 tokens at d = 128, C = 64, bf16) it returns GDR_ERR_TOO_LARGE before
 * enqueuing anything. The stream must belong to the calling thread's current
 * device (else GDR_ERR_LAUNCH).
 *
 * Every call on a GPU shares that GPU's array: calls that may overlap on one
 * GPU (different streams without ordering) race and give wrong results, so
 * order them. Nothing in the array needs clearing between calls (each record
 * is written whole before it is read).
 */
#define GDR_NOALLOC_SCRATCH_BYTES (64u << 20)
int gdr_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                          const void* alpha, const void* b, const void* w,
                          const float* S0, void* o, float* S_out,
                          int B, int H, int T, int dk, int dv, int chunk, int dtype,
                          void* stream);

/*
 * gdr_decode_step — one recurrent step of "Muir: ...", §2.1 eq.(1) for N
 * independent sequences, updating their resident states in place.
 *
 * For each (n, h): with S the state before the call,
 *     S <- (I - k^T (b * k)) Diag(alpha) S + k^T (w * v),   o = q S (new S).
 * It reads S once and writes it once: r = (alpha*b*k) S and p = (alpha*q) S
 * come from one pass, then S <- Diag(alpha) S + k^T (w*v - r) and
 * o = p + (q . k)(w*v - r).
 *
 *   q, k, alpha, b  [N,H,dk]     input dtype
 *   v, w            [N,H,dv]     input dtype
 *   S               [N,H,dk,dv]  float32 state, read and written in place
 *   o               [N,H,dv]     output, input dtype
 * Returns GDR_OK or a negative GDR_ERR_* code.
 */
int gdr_decode_step(const void* q, const void* k, const void* v,
                    const void* alpha, const void* b, const void* w,
                    float* S, void* o,
                    int N, int H, int dk, int dv, int dtype, void* stream);

/*
 * gdr_muir_chunk_fwd_ws, gdr_muir_decode_step — gdr_chunk_fwd_ws and
 * gdr_decode_step with the gate activations of "Muir: Linear Attention with
 * Sensitivity-Allocated Gating and Matched-Filter Readout" folded into the
 * kernels' load stage: the caller passes pre-activation logits instead of the
 * gates, and the gates are formed in float32 from them (§2.1 "Gate
 * Parameterization", §4.1 eq.(9) and the gate list after it, eq.(8)):
 *     log alpha = -exp(a_log[h]) * softplus(z_f),   b = 2 sigmoid(z_b),
 *     w = sigmoid(z_w),   gamma = gamma_stat[h] * 2 sigmoid(z_q),
 * and the recurrence reads out with the gain-modulated query:
 *     S_t = (I - k_t^T (b_t * k_t)) Diag(alpha_t) S_{t-1} + k_t^T (w_t * v_t),
 *     o_t = (gamma_t * q_t) S_t.
 * k stays as given (unit norm on the pages); gamma scales only the readout.
 *
 *   z_f, z_b        [B,H,T,dk] (decode [N,H,dk])  input dtype; decay and erase
 *                   logits (z_f including its bias c_f)
 *   z_w             [B,H,T,dv] (decode [N,H,dv])  input dtype; write logits
 *   z_q             [B,H,T,dk] (decode [N,H,dk])  input dtype; query-gain
 *                   logits, or NULL for z_q = 0 (gamma = gamma_stat: the
 *                   pages' static-gain ablation)
 *   a_log           [H] float32 per-head log-rate (required)
 *   gamma_stat      [H, dk] float32 static readout gain, or NULL for ones
 * a_log and gamma_stat need 4-byte alignment, z_q 16 bytes; outputs must not
 * overlap them. Everything else (shapes, layouts, workspace, state, errors)
 * as for gdr_chunk_fwd_ws and gdr_decode_step.
 */
int gdr_muir_chunk_fwd_ws(const void* q, const void* k, const void* v,
                          const void* z_f, const void* z_b, const void* z_w, const void* z_q,
                          const float* a_log, const float* gamma_stat,
                          const float* S0, void* o, float* S_out,
                          int B, int H, int T, int dk, int dv, int chunk, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream);
int gdr_muir_decode_step(const void* q, const void* k, const void* v,
                         const void* z_f, const void* z_b, const void* z_w, const void* z_q,
                         const float* a_log, const float* gamma_stat,
                         float* S, void* o,
                         int N, int H, int dk, int dv, int dtype, void* stream);

/*
 * gdr_rwkv7_workspace_size, gdr_rwkv7_fwd, gdr_rwkv7_decode_step — RWKV-7's
 * generalized delta rule ("Exponential gates and matrix memory: xLSTM and
 * RWKV-7", §13.3 and the solution to Exercise 13.5) in this library's
 * orientation (state S[dk, dv], row vectors):
 *     S_t = (Diag(w_t) - c_t a_t^T a_t) S_{t-1} + kw_t^T u_t,   o_t = q_t S_t,
 * a per-channel decay w, a unit removal direction a with coefficient c, and a
 * write key kw decoupled from a (the page's b, renamed: it is not GDN-2's
 * erase gate). The removal reads the previous, undecayed state.
 *
 * gdr_rwkv7_fwd runs two kernels through a caller workspace (float32
 * records): every chunk independently (decay-scaled Gram matrices, the unit
 * lower-triangular solve for the removal amounts, and the state-independent
 * parts of the readout and state update), then one pass over the chunks of
 * each head. Every decay factor is exp of a non-positive difference of
 * cumulative log-decays.
 *
 *   q, w, a, kw     [B,H,T,dk]  input dtype (w in (0, 1], a unit)
 *   u               [B,H,T,dv]  input dtype
 *   c               [B,H,T]     float32 removal coefficients
 *   S0, S_out, o    as for gdr_chunk_fwd
 *   chunk           16 or 32 (GDR_ERR_UNSUPPORTED otherwise)
 * gdr_rwkv7_decode_step: one token for N sequences, inputs [N,H,d], c [N,H],
 * S [N,H,dk,dv] updated in place (read once, written once), o [N,H,dv].
 */
int gdr_rwkv7_workspace_size(int B, int H, int T, int dk, int dv, int chunk, size_t* bytes);
int gdr_rwkv7_fwd(const void* q, const void* w, const void* a, const float* c,
                  const void* kw, const void* u, const float* S0, void* o, float* S_out,
                  int B, int H, int T, int dk, int dv, int chunk, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream);
int gdr_rwkv7_decode_step(const void* q, const void* w, const void* a, const float* c,
                          const void* kw, const void* u, float* S, void* o,
                          int N, int H, int dk, int dv, int dtype, void* stream);

/*
 * gdr_mlstm_fwd — chunkwise forward of the xLSTM mLSTM cell with its
 * log-domain stabiliser ("Exponential gates and matrix memory: xLSTM and
 * RWKV-7", §13.4 and Exercise 13.6), in the [dk, dv] orientation:
 *     log f_t = log sigmoid(f_tilde_t),  m_t = max(log f_t + m_{t-1}, i_tilde_t),
 *     C_t = e^{log f_t + m_{t-1} - m_t} C_{t-1} + e^{i_tilde_t - m_t} k_t^T v_t,
 *     n_t = e^{log f_t + m_{t-1} - m_t} n_{t-1} + e^{i_tilde_t - m_t} k_t,
 *     h_t = q_t C_t / max(|q_t . n_t|, e^{-m_t}).
 * Within a chunk the running max is evaluated in its closed form
 * m_t = F_t + max(m_0, max_{s<=t}(i_tilde_s - F_s)), F_t = sum_{r<=t} log f_r,
 * so every exponent is <= 0.
 *
 *   q, k            [B,H,T,dk]  input dtype
 *   v               [B,H,T,dv]  input dtype
 *   i_tilde, f_tilde [B,H,T]    float32 input log-gate and forget-gate logit
 *   C0, n0, m0      [B,H,dk,dv], [B,H,dk], [B,H] float32 initial state; pass
 *                   all three NULL for the empty state (C = 0, n = 0, m = -inf)
 *   h               [B,H,T,dv]  output, input dtype
 *   C_out, n_out, m_out  final state (float32); all NULL to skip. C_out may
 *                   equal C0 (in-place update); n_out and m_out must not
 *                   overlap n0 or m0 (every value tile of a head reads them).
 * Returns GDR_OK or a negative GDR_ERR_* code.
 */
int gdr_mlstm_fwd(const void* q, const void* k, const void* v,
                  const float* i_tilde, const float* f_tilde,
                  const float* C0, const float* n0, const float* m0,
                  void* h, float* C_out, float* n_out, float* m_out,
                  int B, int H, int T, int dk, int dv, int chunk, int dtype,
                  void* stream);

/*
 * gdr_mlstm_workspace_size, gdr_mlstm_fwd_ws — the computation of
 * gdr_mlstm_fwd (same arguments and results up to rounding) as two kernels
 * through a caller workspace, the fast form for long sequences:
 *   1. every (b, h, chunk) in parallel: with F_t, a_s = i~_s - F_s and the
 *      chunk-local running max A_t = max_{s<=t} a_s, the state-independent
 *      parts H_t = sum_{s<=t} e^{a_s - A_t} (q_t . k_s) v_s, its normaliser
 *      N_t (v = 1), K~ = e^{a_s - A_C} k_s, V^T, F and A;
 *   2. one pass over the chunks of each head: mu_t = max(m0, A_t),
 *      h^_t = e^{m0 - mu_t} q_t C0 + e^{A_t - mu_t} H_t (n^ likewise),
 *      h_t = h^_t / max(|n^_t|, e^{-(F_t + mu_t)}),
 *      [C | n] <- e^{m0 - mu_C} [C | n] + e^{A_C - mu_C} K~^T [V | 1],
 *      m <- F_C + mu_C (the stabiliser of §13.4; every exponent <= 0).
 * Record per (b, h, chunk): (2*C*dv + dk*C) elements of the input dtype and
 * 3*C float32, rounded up to 16 bytes; with bfloat16 inputs, d_k and C
 * multiples of 32 and a head's records under 2 GiB, the record also holds
 * a copy of the chunk's q (C*dk elements) and its matrices are stored in
 * MFMA tile order. With few heads and long sequences (bfloat16, C = 64, d_k
 * and d_v multiples of 64, B*H*d_v/64 at most 128, at least 32 chunks) pass 2
 * runs segmented: the chunk map is scalar-decay affine, so a short first
 * segment is scanned beside the end states of the middle segments from a
 * zero start, and the remaining segments then run side by side from the
 * first one's end state with those maps applied; the q copy is then not
 * written (the scan reads q from the input) and the workspace also holds the
 * maps and the first segment's end state (float32). C_out may be C0 on every
 * path. gdr_mlstm_workspace_size reports the size for the given shapes (the
 * plan depends on the shapes only). Workspace rules as for gdr_chunk_fwd_ws.
 * With float32 inputs d_v must be at most 128 here.
 */
int gdr_mlstm_workspace_size(int B, int H, int T, int dk, int dv, int chunk,
                             int dtype, size_t* bytes);
int gdr_mlstm_fwd_ws(const void* q, const void* k, const void* v,
                     const float* i_tilde, const float* f_tilde,
                     const float* C0, const float* n0, const float* m0,
                     void* h, float* C_out, float* n_out, float* m_out,
                     int B, int H, int T, int dk, int dv, int chunk, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable text for a return code (static storage). */
const char* gdr_status_string(int status);

/* Library version: major*10000 + minor*100 + patch. */
int gdr_version(void);

/*
 * gdr_debug_build — 1 for the debug library (GDR_DEBUG defined: every entry
 * point checks its inputs' values, see the top of this header), 0 otherwise.
 *
 * gdr_debug_violation — after an entry point of the debug library returned
 * GDR_ERR_PRECONDITION on the calling thread: the names of the arguments that
 * broke their rule (as in this header, comma-separated; the decays alpha and
 * w must lie in (0, 1], the mLSTM stabiliser m0 may also be -inf, every other
 * input must be finite). "" after a call that passed, and always "" in the
 * release library. The text is thread-local and valid until the thread's
 * next call into the library.
 */
int gdr_debug_build(void);
const char* gdr_debug_violation(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */

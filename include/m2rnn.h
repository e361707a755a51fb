/*
 * m2rnn.h -- C ABI of the MI355X (gfx950) M²RNN recurrence library (libm2rnn.so).
 *
 * The operation is the matrix-state non-linear recurrence of the review of
 * "M²RNN: Non-Linear RNNs with Matrix-Valued States for Scalable Language
 * Modeling" (arXiv:2603.14360v2), section 2.1, Eq. (10)-(12), with the forget
 * gate of the pararnn-torch "ParaM2RNN" page ("Recurrence (library core)":
 * f = sigmoid(logit)) or of the review's section 2.2, Eq. (13)/(17)
 * (f = exp(-alpha * softplus(a + beta))).  Per batch row b and head n, from the
 * initial state H_0 (K x V):
 *
 *     Z_t = tanh(H_{t-1} W_n + k_t v_t^T)          (W_n is V x V, right-multiplied)
 *     H_t = f_t H_{t-1} + (1 - f_t) Z_t
 *     y_t = H_t^T q_t + w_r[n] (.) v_t
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is DEVICE memory owned by the caller, C-contiguous,
 *   in the layout stated next to it, aligned to its element type.  The library
 *   allocates nothing; between calls it keeps only per-device caches of one
 *   occupancy query (m2rnn_step) and of its scratch array's address
 *   (m2rnn_bwd_noalloc), both atomic, so concurrent host threads are safe.
 *   Calls are asynchronous on `stream` (a hipStream_t, NULL = the default
 *   stream) and never synchronise the device.
 * - Wider (16-byte) memory accesses are used where an array's address and row
 *   length allow them and element accesses otherwise, so no alignment beyond
 *   the element type's is required (m2rnn_newton_fwd states its own).
 * - Outputs are overwritten, never accumulated, and must not alias inputs.
 * - `state_dtype` (M2RNN_F32 or M2RNN_F64) is the type of the recurrent state,
 *   of every accumulation, and of every floating-point tensor except k, v, q:
 *   f, logit, alpha, beta, W, w_r, H0, y, HT, ckpt, dy, dHT and every gradient.
 *   F32 is the production path; F64 runs the same kernels in double precision.
 * - `in_dtype` is the type of k, v, q: M2RNN_F32 or M2RNN_BF16 with an F32
 *   state; M2RNN_F64 or M2RNN_BF16 with an F64 state.  bf16 values are widened
 *   exactly.
 * - Arguments are checked on the host before anything is launched; a failed
 *   check returns its status and launches nothing.  Values on the device are
 *   not checked (f in [0, 1], alpha >= 0, finite inputs are preconditions).
 * - Launch failures are reported as M2RNN_ERR_HIP (hipGetLastError).
 * - q and k have `qk_heads` heads shared by groups of n_heads / qk_heads
 *   consecutive value heads: value head n reads q/k head n / (n_heads / qk_heads),
 *   so dq and dk of a shared head sum over its group (the review's section 2.4
 *   multi-value layout is qk_heads = 1; qk_heads = n_heads gives every head its
 *   own q and k).  qk_heads must divide n_heads (1 <= qk_heads <= n_heads; both
 *   are 0 for a call with no heads), else M2RNN_ERR_INVALID_ARG.
 * - Supported sizes: B, T, n_heads >= 0; 1 <= K <= 256; 1 <= V <= 128;
 *   T < 2^30; B * n_heads * ceil(K / 16) < 2^22.  Other sizes return
 *   M2RNN_ERR_UNSUPPORTED (negative ones, or K or V < 1,
 *   M2RNN_ERR_INVALID_ARG).
 * - Empty calls (B, T or n_heads = 0) are defined: nothing is recomputed, the
 *   per-token arrays are empty (their pointers may be NULL), H_T = H_0 (zero
 *   when H0 is NULL), dH_0 = dH_T (zero when dHT is NULL) and dW, dw_r,
 *   dalpha, dbeta are zero (sums over no tokens).  They need no workspace.
 * - Results are bit-reproducible for the same inputs, sizes, device and build
 *   (every reduction runs in a fixed order, without atomics).
 */
#ifndef M2RNN_H_
#define M2RNN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  M2RNN_OK = 0,
  M2RNN_ERR_INVALID_ARG = 1, /* bad size, NULL pointer, bad enum, missing/extra gate parameters */
  M2RNN_ERR_UNSUPPORTED = 2, /* K > 256, V > 128, or an unsupported dtype pairing */
  M2RNN_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than the *_workspace_bytes query */
  M2RNN_ERR_HIP = 4,         /* a kernel launch failed */
  M2RNN_ERR_SCRATCH = 5      /* m2rnn_bwd_noalloc: the call needs more than the static scratch */
} m2rnn_status;

/* Bytes of the static per-device scratch that m2rnn_bwd_noalloc works in. */
#define M2RNN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

typedef enum { M2RNN_F32 = 0, M2RNN_BF16 = 1, M2RNN_F64 = 2 } m2rnn_dtype;

typedef enum { M2RNN_GATE_SIGMOID = 0, M2RNN_GATE_EXP_SOFTPLUS = 1 } m2rnn_gate;

/* Human-readable name of a status code (static storage, never NULL). */
const char* m2rnn_status_string(int status);

/*
 * m2rnn_gates -- forget gate for every (b, t, n) at once.  The gate does not
 * read the state (review section 2.2, last paragraph), so the whole sequence
 * is computed in one elementwise pass.
 *   gate_kind M2RNN_GATE_SIGMOID:      f = 1 / (1 + exp(-logit))       (ParaM2RNN "Recurrence")
 *   gate_kind M2RNN_GATE_EXP_SOFTPLUS: f = exp(-alpha[n] * softplus(logit + beta[n]))
 *                                        = (1 + e^{logit + beta[n]})^{-alpha[n]}   (review Eq. 13/17)
 *   logit  [B, T, n_heads]      in, `dtype` (F32 or F64)
 *   alpha  [n_heads]            in, EXP_SOFTPLUS only, else must be NULL
 *   beta   [n_heads]            in, EXP_SOFTPLUS only, else must be NULL
 *   f      [B, T, n_heads]      out
 */
int m2rnn_gates(int64_t B, int64_t T, int64_t n_heads, int gate_kind, int dtype,
                const void* logit, const void* alpha, const void* beta, void* f,
                void* stream);

/*
 * Workspace (device bytes) that m2rnn_fwd (is_bwd = 0) or m2rnn_bwd
 * (is_bwd = 1) needs for these sizes and checkpoint interval C (C is only
 * used for the backward); 0 means none (workspace may be NULL).  Returns 0 as
 * well for sizes the library rejects.
 */
size_t m2rnn_workspace_bytes(int is_bwd, int64_t B, int64_t T, int64_t n_heads,
                             int64_t qk_heads, int64_t K, int64_t V, int64_t C,
                             int state_dtype);

/*
 * m2rnn_fwd -- the recurrence and readout of review section 2.1, Eq. (10)-(12),
 * for all B * n_heads units, from H0 (or zero), over T steps.
 *   k, q   [B, T, qk_heads, K]  in, in_dtype
 *   v      [B, T, n_heads, V]   in, in_dtype
 *   f      [B, T, n_heads]      in, forget gate (from m2rnn_gates)
 *   W      [n_heads, V, V]      in, (H W)[i][j] = sum_l H[i][l] * W[n][l][j]
 *   w_r    [n_heads, V]         in
 *   H0     [B, n_heads, K, V]   in, or NULL for H_0 = 0
 *   y      [B, T, n_heads, V]   out
 *   HT     [B, n_heads, K, V]   out, final state H_T, or NULL
 *   ckpt   [B, n_heads, ceil(T / C), K, V]  out, ckpt[b][n][c] = H_{cC} (c = 0 is H_0),
 *          or NULL (then C is ignored).  These are the states m2rnn_bwd restarts
 *          from (the review's section 2.6 reruns the recurrence at the start of
 *          the backward; storing every C-th state bounds that rerun to C steps).
 *   C      checkpoint interval, >= 1 when ckpt != NULL
 *   rc     [B, n_heads, T, K, V]  out, or NULL: rc_t = 1 / (1 + e^{2 A_t}) of every step
 *          (A_t the pre-activation, tanh(A_t) = 1 - 2 rc_t).  Given to m2rnn_bwd, it
 *          replaces the backward's recomputation of the states inside each
 *          checkpoint interval (the states follow from rc by the interpolation
 *          alone, bit for bit); it costs K V 4-8 bytes per token and head.
 *   workspace / workspace_bytes: at least m2rnn_workspace_bytes(0, ...)
 */
int m2rnn_fwd(int64_t B, int64_t T, int64_t n_heads, int64_t qk_heads, int64_t K, int64_t V,
              int in_dtype, int state_dtype, const void* k, const void* v, const void* q,
              const void* f, const void* W, const void* w_r, const void* H0, void* y, void* HT,
              void* ckpt, int64_t C, void* rc, void* workspace, size_t workspace_bytes,
              void* stream);

/*
 * m2rnn_bwd -- reverse-time backward of m2rnn_fwd for a loss L with
 * dL/dy = dy and dL/dH_T = dHT, following the corrected chain rule of review
 * section 2.7 (value-residual branch restored).  With u_t = dy_t and C_t the
 * state gradient from later steps (C_T = dHT):
 *     R_t = C_t + q_t u_t^T,   D_t = ((1 - f_t) R_t) (.) (1 - Z_t (.) Z_t),
 *     C_{t-1} = f_t R_t + D_t W^T,
 *     df_t = <R_t, H_{t-1} - Z_t>_F,   dW = sum_{b,t} H_{t-1}^T D_t,
 *     dk_t = D_t v_t,   dv_t = D_t^T k_t + w_r (.) u_t,   dq_t = H_t u_t,
 *     dw_r = sum_{b,t} u_t (.) v_t,   dH0 = C_0,
 * then the gate chain rule: sigmoid: dlogit = df f (1 - f); exp-softplus with
 * x = logit + beta: dlogit = -df alpha sigmoid(x) f, dalpha = sum_{b,t} -df softplus(x) f,
 * dbeta = sum_{b,t} dlogit.  The states are recomputed chunk by chunk from
 * the checkpoints m2rnn_fwd wrote with the same C (review section 2.6).
 *   k, v, q, f, W, w_r, H0     as for m2rnn_fwd (H0 NULL = zero)
 *   gate_kind, logit, alpha, beta   as for m2rnn_gates (alpha/beta NULL for sigmoid)
 *   ckpt   [B, n_heads, ceil(T / C), K, V]  in, from m2rnn_fwd with the same C, H0, inputs
 *   rc     [B, n_heads, T, K, V]  in, from the same m2rnn_fwd call, or NULL to recompute
 *          the states (same results either way)
 *   dy     [B, T, n_heads, V]   in
 *   dHT    [B, n_heads, K, V]   in, or NULL for zero
 *   dk, dq [B, T, qk_heads, K]  out, state_dtype (a shared head's sum over its group)
 *   dv     [B, T, n_heads, V]   out
 *   dlogit [B, T, n_heads]      out, dL/dlogit (sigmoid: g; exp-softplus: a)
 *   dW     [n_heads, V, V]      out, summed over batch and time
 *   dw_r   [n_heads, V]         out, summed over batch and time
 *   dalpha, dbeta [n_heads]     out, EXP_SOFTPLUS only (else must be NULL)
 *   dH0    [B, n_heads, K, V]   out, or NULL to skip
 *   workspace / workspace_bytes: at least m2rnn_workspace_bytes(1, ...), 16-byte aligned
 *          (else M2RNN_ERR_INVALID_ARG).  The kernels walk time in chunks of 4, 2
 *          or 1 steps (by state type and V).  For V > 112, when the chunk is at
 *          least 2 steps and C is a larger multiple of it, at most 1024, the main
 *          kernel sweeps each checkpoint interval once and keeps two intervals of
 *          states (and of rc when recomputing) per 16-row slab here; otherwise,
 *          unless C divides the chunk length, the chunk-start states are
 *          recomputed into it first.
 */
int m2rnn_bwd(int64_t B, int64_t T, int64_t n_heads, int64_t qk_heads, int64_t K, int64_t V,
              int in_dtype, int state_dtype, const void* k, const void* v, const void* q,
              int gate_kind, const void* logit, const void* alpha, const void* beta,
              const void* f, const void* W, const void* w_r, const void* H0, const void* ckpt,
              int64_t C, const void* rc, const void* dy, const void* dHT, void* dk, void* dv,
              void* dq, void* dlogit, void* dW, void* dw_r, void* dalpha, void* dbeta,
              void* dH0, void* workspace, size_t workspace_bytes, void* stream);

/*
 * m2rnn_bwd_noalloc -- m2rnn_bwd for callers that cannot allocate device
 * memory or pass a workspace: code being captured into a HIP graph, tight
 * serving or training loops, harnesses that forbid hipMalloc.  Same arguments,
 * results and checks as m2rnn_bwd, without workspace / workspace_bytes: the
 * kernels work in a fixed array of M2RNN_NOALLOC_SCRATCH_BYTES (64 MiB) that
 * the library holds on each device it runs on until the process ends.  A call
 * whose workspace (m2rnn_workspace_bytes(1, ...)) exceeds that returns
 * M2RNN_ERR_SCRATCH and launches nothing.  The call allocates nothing; its
 * first call on a device looks up that device's array address.  `stream` must
 * belong to the calling thread's current device (else M2RNN_ERR_INVALID_ARG).
 * Every call on a device shares that device's array and leaves its partial
 * sums there (the kernels write every element they read, so nothing needs
 * clearing): calls that may overlap on one device -- on different streams, or
 * from different host threads -- race and must be serialised by the caller.
 */
int m2rnn_bwd_noalloc(int64_t B, int64_t T, int64_t n_heads, int64_t qk_heads, int64_t K,
                      int64_t V, int in_dtype, int state_dtype, const void* k, const void* v,
                      const void* q, int gate_kind, const void* logit, const void* alpha,
                      const void* beta, const void* f, const void* W, const void* w_r,
                      const void* H0, const void* ckpt, int64_t C, const void* rc,
                      const void* dy, const void* dHT, void* dk, void* dv, void* dq,
                      void* dlogit, void* dW, void* dw_r, void* dalpha, void* dbeta, void* dH0,
                      void* stream);

/*
 * m2rnn_step -- one token of every sequence (decoding): the state is updated in
 * place by one step of the recurrence of review section 2.1, Eq. (10)-(12) (the
 * sequential cell step of the pararnn-torch "ParaM2RNN" page), and read out:
 *     H <- f H + (1 - f) tanh(H W_n + k v^T),   y = H^T q + w_r[n] (.) v.
 * Bit-for-bit the same arithmetic as m2rnn_fwd is not promised (the H W sum
 * runs in another order); both are within the library's stated tolerances.
 *   k, q   [B, qk_heads, K]     in, in_dtype
 *   v      [B, n_heads, V]      in, in_dtype
 *   f      [B, n_heads]         in, forget gate (m2rnn_gates with T = 1)
 *   W, w_r                      as for m2rnn_fwd
 *   H      [B, n_heads, K, V]   in/out: H_{t-1} on entry, H_t on return
 *   y      [B, n_heads, V]      out
 * No workspace.  B * n_heads = 0 is a call that reads and writes nothing.
 */
int m2rnn_step(int64_t B, int64_t n_heads, int64_t qk_heads, int64_t K, int64_t V, int in_dtype,
               int state_dtype, const void* k, const void* v, const void* q, const void* f,
               const void* W, const void* w_r, void* H, void* y, void* stream);

/*
 * Parallel-in-time forward by Newton's method (pararnn-torch "ParaM2RNN" page,
 * "Jacobian class" and "Parallel path": factorized Newton on the matrix
 * residual; "ParaGRU" page, "Parallel path": Newton + scan from the guess
 * X_t = F(0, x_t)).  The states X_1 .. X_T of m2rnn_fwd's recurrence are the
 * unknowns; iteration i linearises F(X) = f X + (1 - f) tanh(X W + k v^T) at the
 * current iterate and solves the resulting linear recurrence over time exactly
 * (a two-level scan over chunks, each state row with its own V x V step
 * matrix f I + (1 - f) W diag(1 - Z^2)).  After `iters` iterations the states
 * are read out as in m2rnn_fwd.  The first i states are exact after i
 * iterations (T iterations give the sequential result); the method converges
 * quadratically when every step map is contractive (e.g. |W| < 1) and may
 * diverge otherwise -- `residual` reports max_t |X_t - F(X_{t-1})| of every
 * iterate so that the caller can check.  Its cost per iteration is about
 * V times the sequential forward's flops, spread over all T steps: it pays
 * when B * n_heads * ceil(K / 16) slabs leave most of the device idle.
 *
 * fp32 state only: in_dtype F32 or BF16 (k, v, q); f, W, w_r, H0 and every
 * output fp32.  V must be 16, 32, 48 or 64 (else M2RNN_ERR_UNSUPPORTED); K <= 256;
 * 0 <= iters <= 64.  v, H0, y, HT, states and the workspace must be 16-byte aligned.
 *   k, q, v, f, W, w_r, H0     as for m2rnn_fwd (H0 may be NULL = zeros)
 *   y        [B, T, n_heads, V]      out, the readout of the final iterate
 *   HT       [B, n_heads, K, V]      out or NULL, its last state
 *   states   [B, n_heads, T, K, V]   out or NULL, every state of the final
 *                                    iterate (X_t at index t - 1); when NULL the
 *                                    iterate lives in the workspace
 *   residual [iters + 1]             out or NULL, float: entry i is the largest
 *                                    |X_t - F(X_{t-1})| of iterate i (0 = the guess)
 *   workspace / workspace_bytes: at least m2rnn_newton_workspace_bytes(...)
 * Launches only on `stream`, no allocation.  B * T * n_heads = 0: H_T = H_0
 * (zero when NULL) and residual = 0; nothing else is written.
 */
size_t m2rnn_newton_workspace_bytes(int64_t B, int64_t T, int64_t n_heads, int64_t K, int64_t V,
                                    int states_given);
int m2rnn_newton_fwd(int64_t B, int64_t T, int64_t n_heads, int64_t qk_heads, int64_t K,
                     int64_t V, int in_dtype, const void* k, const void* v, const void* q,
                     const void* f, const void* W, const void* w_r, const void* H0, int iters,
                     void* y, void* HT, void* states, void* residual, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * The block around the recurrence (review section 2.3, Eq. 14-23): q, k, v each
 * pass a linear projection, a depthwise causal Conv1D of kernel size 4 and SiLU
 * (the prologue below); the output gate g = SiLU(W_g x) multiplies the readout,
 * which is then RMS-normalised (the epilogue).  The projections are plain GEMMs
 * and are not part of this library.  For these entry points `io_dtype` (F32,
 * BF16 or F64) is the storage type of x, out and g_pre; `param_dtype` (F32 or
 * F64, paired as for m2rnn_fwd) that of w, bias, gamma, y and every gradient,
 * and the precision of the arithmetic.  bf16 outputs are rounded to nearest
 * even.  Parameter gradients are sums over all tokens, reduced in a fixed order.
 *
 * Workspace of m2rnn_conv_silu_bwd (op 0: x is [B, T, C]) or of
 * m2rnn_gate_rmsnorm_bwd (op 1: rows = B * T, D = C); 0 = none.
 */
size_t m2rnn_block_workspace_bytes(int op, int64_t B, int64_t T, int64_t C, int param_dtype);

/*
 * m2rnn_conv_silu -- prologue on one projected tensor:
 *     out_t[c] = SiLU(u_t[c]),  u_t[c] = bias[c] + sum_{i=0..3} w[c][i] x_{t-3+i}[c],
 * with x_{t<0} = 0 (each sequence starts with no history).
 *   x    [B, T, C]   in, io_dtype
 *   w    [C, 4]      in, param_dtype (tap i weights the input 3 - i steps back)
 *   bias [C]         in, param_dtype, or NULL for none
 *   out  [B, T, C]   out, io_dtype (may feed m2rnn_fwd as k, v or q)
 */
int m2rnn_conv_silu(int64_t B, int64_t T, int64_t C, int io_dtype, int param_dtype,
                    const void* x, const void* w, const void* bias, void* out, void* stream);

/*
 * m2rnn_conv_silu_bwd -- gradients of sum(dout * out):
 *     du = dout SiLU'(u),  dx_s = sum_i w[i] du_{s+3-i},
 *     dw[c][i] = sum_{b,t} du_t[c] x_{t-3+i}[c],  dbias[c] = sum_{b,t} du_t[c].
 *   x, w, bias  as for m2rnn_conv_silu (u is recomputed)
 *   dout [B, T, C]   in, param_dtype (e.g. dk, dv or dq from m2rnn_bwd)
 *   dx   [B, T, C]   out, param_dtype
 *   dw   [C, 4]      out;  dbias [C] out, non-NULL exactly when bias is
 *   workspace / workspace_bytes: at least m2rnn_block_workspace_bytes(0, B, T, C, param_dtype)
 */
int m2rnn_conv_silu_bwd(int64_t B, int64_t T, int64_t C, int io_dtype, int param_dtype,
                        const void* x, const void* w, const void* bias, const void* dout, void* dx,
                        void* dw, void* dbias, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * m2rnn_gate_rmsnorm -- epilogue on the readout of each token:
 *     z = y (.) SiLU(g_pre),  out = gamma (.) z / sqrt(mean_D(z^2) + eps)
 * (gate first, then RMSNorm over the D = n_heads * V channels of the token).
 *   y      [rows, D]   in, param_dtype (m2rnn_fwd's y, rows = B * T)
 *   g_pre  [rows, D]   in, io_dtype (the gate projection W_g x)
 *   gamma  [D]         in, param_dtype
 *   eps    >= 0
 *   out    [rows, D]   out, io_dtype
 */
int m2rnn_gate_rmsnorm(int64_t rows, int64_t D, int io_dtype, int param_dtype, double eps,
                       const void* y, const void* g_pre, const void* gamma, void* out,
                       void* stream);

/*
 * m2rnn_gate_rmsnorm_bwd -- gradients of sum(dout * out): with r = 1 / sqrt(mean(z^2) + eps),
 * zh = z r and dzh = dout gamma:  dz = r (dzh - zh mean_D(dzh zh)),
 * dy = dz SiLU(g_pre),  dg_pre = dz y SiLU'(g_pre),  dgamma = sum_rows dout zh.
 *   y, g_pre, gamma, eps   as for m2rnn_gate_rmsnorm
 *   dout [rows, D]  in, param_dtype;  dy, dg_pre [rows, D] out, param_dtype;  dgamma [D] out
 *   workspace / workspace_bytes: at least m2rnn_block_workspace_bytes(1, rows, 1, D, param_dtype)
 */
int m2rnn_gate_rmsnorm_bwd(int64_t rows, int64_t D, int io_dtype, int param_dtype, double eps,
                           const void* y, const void* g_pre, const void* gamma, const void* dout,
                           void* dy, void* dg_pre, void* dgamma, void* workspace,
                           size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* M2RNN_H_ */

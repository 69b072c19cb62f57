/*
 * linrec.h -- C ABI of the MI355X (gfx950) per-channel linear-recurrence library.
 *
 * Four operations, all over activations laid out (B, T, C) row-major with the channel
 * index fastest (batch B, sequence length T, channels C: the layout the RWKV-LLM page
 * "RWKV：基于RNN的LLM" uses in its section on parallel training):
 *
 *   wkv4_forward / wkv4_backward  the RWKV-4 time-mix operator of eq. (14) on that page
 *   wkv4_forward_ex               the same with a carried state and the sigma(r) gate
 *   wkv4_backward_ex              its backward (gate and carried state)
 *   wkv4_decode_step              one token of it in recurrent form (decoding)
 *   rwkv_token_shift (+ backward) the time-mix token shift of eqs. (11)-(13) feeding it
 *   linrec_scan_real              x_t = a_t * x_{t-1} + b_t (the scan form on the
 *                                 "Were RNNs All We Needed?" news page, minGRU section)
 *   linrec_scan_complex           x_t = lambda * x_{t-1} + u_t (the LRU write-up on
 *                                 "Resurrecting Recurrent Neural Networks for Long
 *                                 Sequences", diagonal complex recurrence, eq. lr-xx)
 *   linrec_scan_real_backward,    the adjoints (backward passes) of the two scans
 *   linrec_scan_complex_backward
 *   linrec_scan_mingru, _minlstm, gated variants of the real scan (minGRU, minLSTM, one decay
 *   _real_decay                   per channel) and the LRU with normalised input, and their
 *   linrec_scan_complex_normalized adjoints (*_backward)
 *
 * Conventions shared by every entry point:
 *  - Pointers are DEVICE pointers (hipMalloc / torch CUDA-on-ROCm memory) unless a
 *    comment says otherwise; the caller owns every buffer for the whole call.  Outputs
 *    must not alias inputs or each other (the one exception: the state of
 *    wkv4_decode_step, updated in place).
 *  - Calls are asynchronous: they validate arguments on the host, then enqueue kernels on
 *    `stream` (a hipStream_t; NULL means the default stream) and return.  The library never
 *    synchronises, allocates or frees device memory; scratch memory comes from the
 *    caller's `workspace` of at least the size the matching *_workspace_size query returns
 *    for the same (B, T, C).  A size of 0 needs no workspace (NULL is then allowed).
 *  - Each call stamps its workspace's look-back flags with a tag drawn on the host at call
 *    time, so stale flags of earlier calls read as unpublished and the workspace needs no
 *    clearing.  A call made while `stream` is capturing into a HIP graph keeps its tag on
 *    every replay, so it also records a fill kernel that clears its flags before its own
 *    kernels: each replay of the graph computes afresh (replays see the workspace and
 *    buffers captured with the call).  Two calls in flight at the same time must not share
 *    a workspace.
 *  - Return value: LINREC_OK or an error status.  Argument checks run before any HIP call:
 *      B, T or C negative, or B*T*C*element size overflowing int64
 *                                                         -> LINREC_ERR_INVALID_ARG
 *      any of B, T, C equal to 0                          -> LINREC_OK, nothing enqueued and
 *        no pointer read, except that the gradient sums over an empty batch or sequence
 *        are zero-filled: gw, gu (wkv4_backward, and gs_in passed through by
 *        wkv4_backward_ex) and glambda (the complex, real-decay and normalised-LRU
 *        backwards) when C > 0, and gx0 of the scan backwards when given and B, C > 0
 *      a required pointer NULL (for a non-empty shape)    -> LINREC_ERR_INVALID_ARG
 *      ws_bytes below the workspace size                  -> LINREC_ERR_WORKSPACE
 *      a pointer not aligned to its element size (4 B for float, 8 B for complex64)
 *        or a workspace not aligned to 16 B               -> LINREC_ERR_UNSUPPORTED
 *      a failed kernel launch                             -> LINREC_ERR_HIP
 *    linrec_last_error() then holds a readable message (per thread).  Faults that happen
 *    while kernels run surface on the stream, as for any HIP work.
 *  - Input values are not inspected (that would need a device read): non-finite inputs
 *    propagate to the outputs.
 *  - Arithmetic is float32 (complex64 as float32 pairs); results match an fp64 evaluation
 *    of the same definition to a relative error of about 1e-5 of the per-sequence RMS.
 */
#ifndef LINREC_H
#define LINREC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LINREC_ABI_VERSION 1

typedef enum {
    LINREC_OK = 0,
    LINREC_ERR_INVALID_ARG = 1,
    LINREC_ERR_WORKSPACE = 2,
    LINREC_ERR_UNSUPPORTED = 3,
    LINREC_ERR_HIP = 4
} linrec_status;

/* Version of this ABI (LINREC_ABI_VERSION of the library that was built). */
int linrec_abi_version(void);

/* Static name of a status code ("LINREC_OK", ...); "unknown status" otherwise. */
const char *linrec_status_string(int status);

/* Detail of the last failing call on the calling thread ("" if none).  The pointer stays
 * valid until the next library call on the same thread. */
const char *linrec_last_error(void);

/* Bytes of device workspace each operation needs for a given shape (0 when none).  Pure
 * host functions of (B, T, C); they make no HIP call.  Negative sizes return 0. */
size_t wkv4_forward_workspace_size(int64_t B, int64_t T, int64_t C);
size_t wkv4_backward_workspace_size(int64_t B, int64_t T, int64_t C);
/* is_complex: 0 for linrec_scan_real and its gated variants, 1 for linrec_scan_complex and
 * linrec_scan_complex_normalized; the backward query likewise covers every adjoint of the
 * family (the plain scan's and its variants'). */
size_t linrec_scan_workspace_size(int64_t B, int64_t T, int64_t C, int is_complex);
size_t linrec_scan_backward_workspace_size(int64_t B, int64_t T, int64_t C, int is_complex);

/*
 * WKV-4 forward, RWKV-LLM page, section "Time-mixing block", eq. (14).  For each batch
 * row b and channel c, with time starting at 0 and an empty past at t = 0:
 *
 *   y[b,t,c] = ( sum_{i<t} e^{-(t-1-i) w[c] + k[b,i,c]} v[b,i,c] + e^{u[c]+k[b,t,c]} v[b,t,c] )
 *            / ( sum_{i<t} e^{-(t-1-i) w[c] + k[b,i,c]}          + e^{u[c]+k[b,t,c]} )
 *
 *   w  (C)      float32, per-channel decay, finite and >= 0 (eq. (10)'s requirement)
 *   u  (C)      float32, per-channel bonus for the current token
 *   k, v (B,T,C) float32 inputs;  y (B,T,C) float32 output
 *
 * Evaluated with a running maximum of the exponents, so no e^{k} is ever formed:
 * k of any magnitude that keeps the sums meaningful in float32 is fine.
 */
int wkv4_forward(int64_t B, int64_t T, int64_t C,
                 const float *w, const float *u, const float *k, const float *v,
                 float *y, void *workspace, size_t ws_bytes, void *stream);

/*
 * WKV-4 forward with a carried state and the receptance gate, for sequences processed in
 * pieces (and token-by-token decoding, T = 1) and for the time-mix output of eq. (15) on
 * the RWKV-LLM page ("Time-mixing block"), o_t = W_o (sigma(r_t) (.) wkv_t) before W_o:
 *
 *   state (a, b, p) per (batch row, channel): the past sums of eq. (14) over every token
 *   already consumed, A = a e^p and B = b e^p, so that the call's first token sees
 *   y_0 = sigma(r_0) (A + e^{u+k_0} v_0) / (B + e^{u+k_0});  a = b = 0 is the empty state.
 *
 *   r     (B,T,C) float32 or NULL (no gate: sigma = 1)
 *   s_in  (B,C,3) float32 (a, b, p) or NULL (empty state)
 *   y     (B,T,C) float32 output
 *   s_out (B,C,3) float32 or NULL: the state after the last token, ready to be the next
 *         call's s_in (its p is chosen by the library; with T = 0 it is s_in, or empty)
 *
 * Same workspace as wkv4_forward.  With T = 0 only s_in and s_out are used.
 */
int wkv4_forward_ex(int64_t B, int64_t T, int64_t C,
                    const float *w, const float *u, const float *k, const float *v,
                    const float *r, const float *s_in, float *y, float *s_out,
                    void *workspace, size_t ws_bytes, void *stream);

/*
 * Token shift of the RWKV time-mix block (RWKV-LLM page, section "Time-mixing block", eqs.
 * (11)-(13)): the inputs of the r, k and v projections interpolate per channel between the
 * current token and the previous one,
 *
 *   out[m,b,t,c] = mu[m,c] * x[b,t,c] + (1 - mu[m,c]) * x[b,t-1,c],    m = 0 .. M-1,
 *
 * with x[b,-1,c] = x_prev[b,c], or 0 when x_prev is NULL.  One call reads x once and writes
 * all M mixes (M = 3 for the time mix's r, k, v; 2 for the channel mix's r, k).
 *
 *   x      (B,T,C) float32;  x_prev (B,C) float32 or NULL (the last token of an earlier
 *          call, for sequences processed in pieces)
 *   mu     (M,C) float32, 1 <= M <= 4
 *   out    (M,B,T,C) float32 output, mix m at out + m*B*T*C
 *
 * No workspace.  M outside 1..4 -> LINREC_ERR_INVALID_ARG.
 */
int rwkv_token_shift(int64_t B, int64_t T, int64_t C, int64_t M, const float *x, const float *x_prev,
                     const float *mu, float *out, void *stream);

/*
 * Backward of rwkv_token_shift (chain rule; the pages give none).  Given g = dL/dout
 * (M,B,T,C):
 *
 *   gx[b,t,c]    = sum_m mu[m,c] g[m,b,t,c] + (1 - mu[m,c]) g[m,b,t+1,c]   (no t+1 term at T-1)
 *   gmu[m,c]     = sum over b and t of g[m,b,t,c] (x[b,t,c] - x[b,t-1,c])
 *   gx_prev[b,c] = sum_m (1 - mu[m,c]) g[m,b,0,c]
 *
 *   x, x_prev, mu as for the forward;  gx (B,T,C), gmu (M,C) float32 outputs;
 *   gx_prev (B,C) float32 output or NULL.
 *
 * gmu is summed in float64 in a fixed order (results do not depend on scheduling) and
 * needs rwkv_token_shift_backward_workspace_size(B, T, C, M) bytes of workspace.  With B or
 * T = 0, gmu (and gx_prev when B > 0) are zero-filled.
 */
size_t rwkv_token_shift_backward_workspace_size(int64_t B, int64_t T, int64_t C, int64_t M);
int rwkv_token_shift_backward(int64_t B, int64_t T, int64_t C, int64_t M, const float *x,
                              const float *x_prev, const float *mu, const float *g, float *gx,
                              float *gmu, float *gx_prev, void *workspace, size_t ws_bytes,
                              void *stream);

/*
 * One token of WKV-4 in its recurrent form, for token-by-token decoding (the RNN mode of
 * inference on the RWKV pages: the output depends only on the current input and a state of
 * fixed size; RWKV-LLM page, "并行训练和序列解码"):
 *
 *   y     = sigma(r) (A + e^{u+k} v) / (B + e^{u+k})         (eqs. (14)-(15) at one step)
 *   state <- (e^{-w} A + e^{k} v,  e^{-w} B + e^{k})
 *
 *   w, u  (C)     float32 as for wkv4_forward
 *   k, v  (B,C)   float32, this token of each batch row
 *   r     (B,C)   float32 or NULL (no gate: sigma = 1)
 *   state (B,C,3) float32 (a, b, p), A = a e^p and B = b e^p, read and then OVERWRITTEN IN
 *                 PLACE with the state after this token (the one buffer that is both input
 *                 and output); a = b = 0 is the empty state.  Interchangeable with the
 *                 s_in / s_out of wkv4_forward_ex.
 *   y     (B,C)   float32 output
 *
 * No workspace.  Calling it T times gives wkv4_forward_ex's outputs and final state for the
 * same T tokens (to rounding).
 */
int wkv4_decode_step(int64_t B, int64_t C, const float *w, const float *u, const float *k,
                     const float *v, const float *r, float *state, float *y, void *stream);

/*
 * WKV-4 backward: given the upstream gradient gy = dL/dy of eq. (14)'s output, writes
 *
 *   gw (C), gu (C)     dL/dw and dL/du, summed over batch and time (w and u are
 *                      per-channel vectors in eq. (14)); w as it appears in eq. (14),
 *                      not a log-parametrisation
 *   gk, gv (B,T,C)     dL/dk and dL/dv
 *
 * The pages give no backward pass; these are the chain-rule derivatives of eq. (14).
 * All four outputs are overwritten (not accumulated).  Deterministic: the batch
 * reduction of gw and gu runs in a fixed order.
 */
int wkv4_backward(int64_t B, int64_t T, int64_t C,
                  const float *w, const float *u, const float *k, const float *v,
                  const float *gy, float *gw, float *gu, float *gk, float *gv,
                  void *workspace, size_t ws_bytes, void *stream);

/*
 * Backward of wkv4_forward_ex: the gated time-mix output o_t = sigma(r_t) wkv_t (RWKV-LLM
 * page, eq. (15), before W_o) over a sequence that may start from a carried state and
 * whose final state may feed a later call.  Given gy = dL/do it writes the gradients of
 * wkv4_backward for dL/dwkv_t = gy_t sigma(r_t), and
 *
 *   gr    (B,T,C) float32 output:  dL/dr_t = gy_t wkv_t sigma(r_t) (1 - sigma(r_t))
 *   gs_in (B,C,2) float32 output:  dL/da, dL/db of s_in = (a, b, p), its p held fixed
 *
 *   r      (B,T,C) float32, as given to the forward; r and gr are given together (both NULL:
 *                  no gate, sigma = 1), otherwise LINREC_ERR_INVALID_ARG
 *   s_in   (B,C,3) float32 (a, b, p) as given to the forward, or NULL (empty state)
 *   s_out  (B,C,3) float32, the forward's s_out; only its p is read, and only with gs_out
 *   gs_out (B,C,2) float32 dL/d(a', b') of s_out = (a', b', p') with p' held fixed, or NULL
 *                  (the final state not used); given without s_out: LINREC_ERR_INVALID_ARG
 *   gs_in  may be NULL (not wanted)
 *
 * With p fixed, A = a e^p gives dL/dA = (dL/da) e^{-p}: the final state's gradient enters the
 * reverse sums as dL/dA_T, dL/dB_T, and dL/dw gains their share.  Calls chained through the
 * state (s_out of one as s_in of the next) chain their gradients the same way: the gs_in of
 * the later call is the gs_out of the earlier one.  The pages give no backward; this is the
 * chain rule of eq. (14) with the state as its sums before the first token.  T = 0: the
 * state passes through, gs_in = gs_out e^{p_in - p_out} (zero without gs_out), gw = gu = 0.
 * Same workspace as wkv4_backward.
 */
int wkv4_backward_ex(int64_t B, int64_t T, int64_t C,
                     const float *w, const float *u, const float *k, const float *v,
                     const float *r, const float *s_in, const float *s_out, const float *gy,
                     const float *gs_out, float *gw, float *gu, float *gk, float *gv, float *gr,
                     float *gs_in, void *workspace, size_t ws_bytes, void *stream);

/*
 * Checkpointed training step of WKV-4 (eq. (14); the pages give no backward, whose chain
 * rule needs the forward sums A, B and their derivatives A', B' in w at every step).
 * wkv4_backward recomputes, in a pass of its own over k and v, those sums at the start of
 * every slab of its gradient kernel.  A forward that is
 * followed by a backward can keep those sums instead:
 *
 *   wkv4_forward_ckpt   writes y exactly as wkv4_forward (to rounding), and the sums at the
 *                       end of every slab into ckpt;
 *   wkv4_backward_ckpt  writes gw, gu, gk, gv exactly as wkv4_backward (to rounding) from
 *                       the same w, u, k, v, gy and that ckpt, without the extra pass.
 *   (The sums do not depend on r: one ckpt serves the gated and the plain backward.)
 *
 *   ckpt  device buffer of at least wkv4_checkpoint_size(B, T, C) bytes, 16-byte aligned,
 *         owned by the caller.  Its contents are opaque (float32 mantissas of the sums with
 *         an integer exponent, 20 bytes per channel and slab); they are valid only for the
 *         B, T, C, w and k, v of
 *         the forward that wrote them, and only after that forward has completed in stream
 *         order.  The backward only reads it.
 *   r     (B,T,C) float32 receptance, or NULL: with r the output is the gated sigma(r) wkv
 *         (eq. (15)), as wkv4_forward_ex / wkv4_backward_ex with r, and the backward writes
 *   gr    (B,T,C) dL/dr; r and gr are given together to the backward (else INVALID_ARG)
 *   other arguments as for wkv4_forward / wkv4_backward.  For a carried state see
 *   wkv4_forward_ckpt_ex / wkv4_backward_ckpt_ex below.
 *
 * Workspaces: wkv4_forward_ckpt_workspace_size and wkv4_backward_ckpt_workspace_size (the
 * latter smaller than wkv4_backward's: no state pass).  Errors as for the other calls, and
 * a ckpt smaller than wkv4_checkpoint_size -> LINREC_ERR_WORKSPACE, NULL -> INVALID_ARG,
 * misaligned -> UNSUPPORTED.  B, T or C = 0: the forward does nothing; the backward
 * zero-fills gw and gu (when C > 0).  The slab length of the checkpoints is fixed by the
 * library (56 steps) and does not follow the tuning overrides of the plain calls.
 */
size_t wkv4_checkpoint_size(int64_t B, int64_t T, int64_t C);
size_t wkv4_forward_ckpt_workspace_size(int64_t B, int64_t T, int64_t C);
size_t wkv4_backward_ckpt_workspace_size(int64_t B, int64_t T, int64_t C);
int wkv4_forward_ckpt(int64_t B, int64_t T, int64_t C,
                      const float *w, const float *u, const float *k, const float *v,
                      const float *r, float *y, void *ckpt, size_t ckpt_bytes,
                      void *workspace, size_t ws_bytes, void *stream);
int wkv4_backward_ckpt(int64_t B, int64_t T, int64_t C,
                       const float *w, const float *u, const float *k, const float *v,
                       const float *r, const float *gy, const void *ckpt, size_t ckpt_bytes,
                       float *gw, float *gu, float *gk, float *gv, float *gr,
                       void *workspace, size_t ws_bytes, void *stream);

/*
 * The checkpointed training step for a sequence processed in pieces (RWKV-LLM page, section
 * "并行训练和序列解码": the recurrence carries a state from one piece to the next): as
 * wkv4_forward_ckpt / wkv4_backward_ckpt, with the carried state of wkv4_forward_ex /
 * wkv4_backward_ex.
 *
 *   wkv4_forward_ckpt_ex   starts from s_in (B,C,3) (a, b, p) or NULL (empty state), writes
 *                          y, the kept sums (which then include the state) and, when s_out
 *                          is not NULL, the state after the last token (B,C,3);
 *   wkv4_backward_ckpt_ex  takes the same s_in, the forward's s_out (only its p is read, and
 *                          only with gs_out), gs_out = dL/d(a', b') of s_out (B,C,2) or NULL,
 *                          and writes gs_in = dL/d(a, b) of s_in (B,C,2) when not NULL; the
 *                          gradients are those of wkv4_backward_ex (to rounding), from the
 *                          ckpt its forward wrote for the same w, k, v and s_in.
 *
 * Calls chained through the state chain their gradients as wkv4_backward_ex's do (the gs_in
 * of a later piece is the gs_out of the earlier one).  T = 0: the forward passes the state
 * through (s_out = s_in, or empty) and writes no checkpoint; the backward writes gw = gu = 0
 * and gs_in = gs_out e^{p_in - p_out}.  Sizes, workspaces and errors as for the calls above,
 * plus: gs_out without s_out -> LINREC_ERR_INVALID_ARG; a state pointer not 4-byte aligned
 * -> LINREC_ERR_UNSUPPORTED.
 */
int wkv4_forward_ckpt_ex(int64_t B, int64_t T, int64_t C,
                         const float *w, const float *u, const float *k, const float *v,
                         const float *r, const float *s_in, float *y, float *s_out,
                         void *ckpt, size_t ckpt_bytes, void *workspace, size_t ws_bytes, void *stream);
int wkv4_backward_ckpt_ex(int64_t B, int64_t T, int64_t C,
                          const float *w, const float *u, const float *k, const float *v,
                          const float *r, const float *s_in, const float *s_out, const float *gy,
                          const float *gs_out, const void *ckpt, size_t ckpt_bytes,
                          float *gw, float *gu, float *gk, float *gv, float *gr, float *gs_in,
                          void *workspace, size_t ws_bytes, void *stream);

/*
 * Real diagonal scan, "Were RNNs All We Needed?" page, minGRU section (v_t = a_t (.)
 * v_{t-1} + b_t):  x[b,t,c] = a[b,t,c] * x[b,t-1,c] + b[b,t,c],  x[b,-1,c] = x0[b,c].
 *
 *   a, b (B,T,C) float32;  x0 (B,C) float32 or NULL for a zero initial state;
 *   x (B,T,C) float32 output.  minGRU's h_t = (1-z_t) h_{t-1} + z_t h~_t is a = 1-z,
 *   b = z * h~.
 */
int linrec_scan_real(int64_t B, int64_t T, int64_t C,
                     const float *a, const float *b, const float *x0, float *x,
                     void *workspace, size_t ws_bytes, void *stream);

/*
 * Complex diagonal scan, LRU write-up, section on the diagonal complex recurrence
 * (eq. lr-xx):  x[b,t,c] = lambda[c] * x[b,t-1,c] + u[b,t,c],  x[b,-1,c] = x0[b,c].
 *
 *   lambda (C) complex64 as interleaved (re, im) float pairs, |lambda| <= 1 expected
 *   u (B,T,C) complex64;  x0 (B,C) complex64 or NULL for zero (then x_0 = u_0, as in the
 *   write-up's unrolled form eq. lr-e);  x (B,T,C) complex64 output.
 *
 * Chunk multipliers lambda^n are formed in float64 from the given complex64 lambda.
 */
int linrec_scan_complex(int64_t B, int64_t T, int64_t C,
                        const float *lambda, const float *u, const float *x0, float *x,
                        void *workspace, size_t ws_bytes, void *stream);

/*
 * Gated variants of linrec_scan_real: the coefficients are formed from the gates inside the
 * kernel, so a and b never travel through memory.  All take x0 (B,C) float32 or NULL (zero),
 * write x (B,T,C) float32, and need linrec_scan_workspace_size(B, T, C, 0) bytes of
 * workspace.  Inputs are float32 (B,T,C) unless marked (C).
 *
 * linrec_scan_mingru (minGRU page, minGRU section; its equations are images, read as)
 *     z_t = sigmoid(kz_t),   x_t = (1 - z_t) x_{t-1} + z_t h_t      (h: the candidate h~)
 * linrec_scan_minlstm (minGRU page, minLSTM section: the two gates are normalised)
 *     f_t = sigmoid(kf_t), i_t = sigmoid(ki_t),
 *     x_t = f_t / (f_t + i_t) x_{t-1} + i_t / (f_t + i_t) h_t
 *     (evaluated through log-gate differences: finite for any finite kf, ki)
 * linrec_scan_real_decay (one decay per channel: an SLRU, LRU write-up, section on RWKV)
 *     x_t = lambda[c] x_{t-1} + u_t,   lambda (C)
 */
int linrec_scan_mingru(int64_t B, int64_t T, int64_t C, const float *kz, const float *h,
                       const float *x0, float *x, void *workspace, size_t ws_bytes, void *stream);
int linrec_scan_minlstm(int64_t B, int64_t T, int64_t C, const float *kf, const float *ki,
                        const float *h, const float *x0, float *x, void *workspace,
                        size_t ws_bytes, void *stream);
int linrec_scan_real_decay(int64_t B, int64_t T, int64_t C, const float *lambda, const float *u,
                           const float *x0, float *x, void *workspace, size_t ws_bytes,
                           void *stream);

/*
 * The LRU with normalised input (LRU write-up, initialisation section: a stationary input
 * of variance s feeds a state of variance s / (1 - |lambda|^2), so the input is scaled to
 * keep the state's scale):
 *
 *   x_t = lambda x_{t-1} + gamma u_t,   gamma[c] = sqrt(max(0, 1 - |lambda[c]|^2))
 *
 * Arguments, layout and workspace as linrec_scan_complex.  The method's domain is
 * |lambda| <= 1 (the write-up's r in [0, 1]); |lambda|^2 is formed in double from the
 * complex64 components, and where it exceeds 1 (a unit-modulus lambda rounded to
 * complex64 often does) gamma is 0, its value at r = 1.  Values are not checked: a lambda
 * well outside the unit disc is also scanned with gamma = 0.
 */
int linrec_scan_complex_normalized(int64_t B, int64_t T, int64_t C, const float *lambda,
                                   const float *u, const float *x0, float *x, void *workspace,
                                   size_t ws_bytes, void *stream);

/*
 * Adjoint of linrec_scan_real (the pages give no backward; this is the chain rule of the
 * scan form).  Given the forward output x and the upstream gradient gx = dL/dx, runs
 * backwards in time
 *
 *   gb[b,t,c] = gx[b,t,c] + a[b,t+1,c] * gb[b,t+1,c]      (gb[b,T-1,c] = gx[b,T-1,c])
 *   ga[b,t,c] = gb[b,t,c] * x[b,t-1,c]                    (x[b,-1,c] = x0[b,c], or 0)
 *   gx0[b,c]  = a[b,0,c] * gb[b,0,c]
 *
 *   a, x, gx (B,T,C) float32 inputs (x: the forward output for these a, b, x0);
 *   x0 (B,C) float32 or NULL (zero);  ga, gb (B,T,C) float32 outputs (dL/da, dL/db);
 *   gx0 (B,C) float32 output or NULL when the initial state's gradient is not wanted.
 */
int linrec_scan_real_backward(int64_t B, int64_t T, int64_t C,
                              const float *a, const float *x0, const float *x, const float *gx,
                              float *ga, float *gb, float *gx0,
                              void *workspace, size_t ws_bytes, void *stream);

/*
 * Adjoint of linrec_scan_complex, for a real loss L with complex gradients taken as
 * dL/dRe + i dL/dIm (so that dL = Re sum conj(g) dz).  Backwards in time:
 *
 *   gu[b,t,c]  = gx[b,t,c] + conj(lambda[c]) * gu[b,t+1,c]
 *   glambda[c] = sum over b and t of gu[b,t,c] * conj(x[b,t-1,c])   (x[b,-1,c] = x0 or 0)
 *   gx0[b,c]   = conj(lambda[c]) * gu[b,0,c]
 *
 *   lambda (C), x, gx (B,T,C) complex64 inputs (x: the forward output);  x0 (B,C) or NULL;
 *   glambda (C) complex64 output, summed over batch and time in a fixed order;
 *   gu (B,T,C) complex64 output (dL/du);  gx0 (B,C) complex64 output or NULL.
 */
int linrec_scan_complex_backward(int64_t B, int64_t T, int64_t C,
                                 const float *lambda, const float *x0, const float *x,
                                 const float *gx, float *glambda, float *gu, float *gx0,
                                 void *workspace, size_t ws_bytes, void *stream);

/*
 * Adjoints of the gated variants (chain rule of their forward forms; the pages give no
 * backward).  Each runs backwards in time like linrec_scan_real_backward, with the
 * multiplier a_{t+1} formed from the gates, and d_t = dL/dx_t (all paths):
 *
 *   d_t = gx_t + a_{t+1} d_{t+1}                                  (no carry at T-1)
 *
 * minGRU (a = 1 - z, z = sigmoid(kz)):
 *   gkz_t = d_t z_t (1 - z_t) (h~_t - x_{t-1}),  gh_t = d_t z_t,  gx0 = (1 - z_0) d_0
 * minLSTM (a = f/(f+i), f = sigmoid(kf), i = sigmoid(ki); ga_t = d_t (x_{t-1} - h~_t)):
 *   gkf_t = ga_t a (1 - a) (1 - f),  gki_t = -ga_t a (1 - a) (1 - i),  gh_t = d_t (1 - a_t),
 *   gx0 = a_0 d_0
 * per-channel decay (a = lambda[c]):
 *   gu_t = d_t,  glambda[c] = sum over b and t of d_t x_{t-1},  gx0 = lambda d_0
 *
 * x_{-1} = x0 or 0.  Inputs as for the forward call plus x (B,T,C), the forward's output for
 * the same inputs, and gx (B,T,C) = dL/dx; outputs (B,T,C) float32 gkz, gh / gkf, gki, gh /
 * gu; glambda (C) float32 (summed in float64 in a fixed order); gx0 (B,C) or NULL.
 * Workspace: linrec_scan_backward_workspace_size(B, T, C, 0).  With B or T = 0, glambda and
 * gx0 are zero-filled.
 */
int linrec_scan_mingru_backward(int64_t B, int64_t T, int64_t C, const float *kz, const float *h,
                                const float *x0, const float *x, const float *gx, float *gkz, float *gh,
                                float *gx0, void *workspace, size_t ws_bytes, void *stream);
int linrec_scan_minlstm_backward(int64_t B, int64_t T, int64_t C, const float *kf, const float *ki,
                                 const float *h, const float *x0, const float *x, const float *gx, float *gkf,
                                 float *gki, float *gh, float *gx0, void *workspace, size_t ws_bytes,
                                 void *stream);
int linrec_scan_real_decay_backward(int64_t B, int64_t T, int64_t C, const float *lambda, const float *x0,
                                    const float *x, const float *gx, float *glambda, float *gu, float *gx0,
                                    void *workspace, size_t ws_bytes, void *stream);

/*
 * Adjoint of linrec_scan_complex_normalized (complex gradients as dL/dRe + i dL/dIm), with
 * s_t the adjoint of linrec_scan_complex_backward (s_t = gx_t + conj(lambda) s_{t+1}):
 *
 *   gu_t    = gamma s_t,   gx0 = conj(lambda) s_0,
 *   glambda = sum of s_t conj(x_{t-1}) - (sum of Re(conj(s_t) u_t) / gamma) lambda
 *
 * (gamma = sqrt(max(0, 1 - |lambda|^2)) as in the forward; the second term is dL/dgamma
 * times gamma's gradient, taken as 0 where gamma = 0, where gamma has no derivative).
 * u (B,T,C) complex64 is the forward's input; the rest as
 * linrec_scan_complex_backward.  Workspace: linrec_scan_backward_workspace_size(B, T, C, 1).
 */
int linrec_scan_complex_normalized_backward(int64_t B, int64_t T, int64_t C, const float *lambda,
                                            const float *u, const float *x0, const float *x,
                                            const float *gx, float *glambda, float *gu, float *gx0,
                                            void *workspace, size_t ws_bytes, void *stream);

/*
 * wkv4_forward without a workspace argument, for callers that cannot allocate device memory
 * or pass a workspace: code being captured into a HIP graph, tight serving loops, harnesses
 * that forbid allocation.  It computes exactly what wkv4_forward computes (the same kernels);
 * the look-back flags and records those kernels need live in a static device array of
 * LINREC_NOALLOC_SCRATCH_BYTES that the library keeps on every GPU it runs on until the
 * process ends.  The call allocates and frees nothing.
 *
 *   arguments as wkv4_forward, without workspace / ws_bytes;
 *   a call whose launch needs more scratch than the array holds (e.g. B=8 T=1024 C=768 needs
 *   about 1.2 MB, B=8 T=4096 C=2560 about 15.8 MB) returns LINREC_ERR_UNSUPPORTED before any
 *   HIP call; use wkv4_forward with a workspace for those;
 *   calls on one GPU share its array: two calls that may run at the same time on one GPU
 *   (different streams, or different host threads on different streams) race and must be
 *   ordered by the caller.  Calls in sequence on one stream are safe: the flags carry a
 *   per-call tag, so an earlier call's records never read as this call's.
 *   The first call on each device looks up the array's address there (hipGetSymbolAddress,
 *   with that device current); a failure is LINREC_ERR_HIP.
 */
#define LINREC_NOALLOC_SCRATCH_BYTES (16u * 1024u * 1024u)
int wkv4_forward_noalloc(int64_t B, int64_t T, int64_t C,
                         const float *w, const float *u, const float *k, const float *v,
                         float *y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LINREC_H */

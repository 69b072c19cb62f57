/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.  Plain, slow, fp64 CPU reference of the
 * per-channel linear recurrences.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this; the product path never does.  It shares no code,
 * header, constant or helper with the HIP library.
 *
 * Every routine reads the same float32 / complex64 arrays the GPU receives, widens
 * them exactly to double, and evaluates the definition one channel at a time, time
 * step by time step, in IEEE double with libm's exp (no fast-math).  Channels are
 * independent, so OpenMP splits the (batch, channel) pairs over threads; each pair's
 * arithmetic is the same sequence whatever the thread count, and the per-channel
 * gradient sums over the batch are added in ascending batch order afterwards, so
 * the results do not depend on the number of threads.
 *
 * Layout: (B,T,C) row-major, C fastest; per-channel vectors are (C,); complex
 * values are interleaved (re, im) pairs.
 *
 * Valid range: the WKV routines rescale every channel by exp(-max_t k_t), which
 * cancels exactly in the ratio; they need the per-channel spread of k below ~700
 * and |u| below ~300 so that no used weight underflows double precision.
 */
#include <complex.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static double chan_max_k(const float *k, int64_t T, int64_t C, int64_t base)
{
    double m = -INFINITY;
    for (int64_t t = 0; t < T; ++t) {
        double kt = (double)k[base + t * C];
        if (kt > m) m = kt;
    }
    return m;
}

/*
 * WKV-4 forward.  RWKV-LLM page ("RWKV：基于RNN的LLM"), section "Time-mixing block",
 * eq. (14): for one channel with decay w >= 0 and bonus u,
 *
 *   y_t = ( sum_{i<t} e^{-(t-1-i)w + k_i} v_i + e^{u+k_t} v_t )
 *       / ( sum_{i<t} e^{-(t-1-i)w + k_i}     + e^{u+k_t}     ),
 *
 * with the time index starting at 0 and an empty past at t = 0 (so y_0 = v_0).
 * The two past sums obey A_{t+1} = e^{-w} A_t + e^{k_t} v_t and
 * B_{t+1} = e^{-w} B_t + e^{k_t} (the "two SLRU" reading in the LRU write-up's section
 * on RWKV), which is how they are accumulated here.  All exponentials are taken
 * relative to K = max_t k_t; the common factor e^{-K} cancels in the ratio.
 */
void oracle_wkv4_forward(int64_t B, int64_t T, int64_t C,
                         const float *w, const float *u,
                         const float *k, const float *v, double *y)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t bc = 0; bc < B * C; ++bc) {
        const int64_t b = bc / C, c = bc % C;
        const int64_t base = b * T * C + c;
        const double K = chan_max_k(k, T, C, base);
        const double decay = exp(-(double)w[c]);
        const double uu = (double)u[c];
        double A = 0.0, Bs = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const int64_t o = base + t * C;
            const double kt = (double)k[o], vt = (double)v[o];
            const double cur = exp(uu + kt - K);   /* e^{u+k_t}, rescaled */
            y[o] = (A + cur * vt) / (Bs + cur);
            const double past = exp(kt - K);       /* e^{k_t}, rescaled */
            A = decay * A + past * vt;
            Bs = decay * Bs + past;
        }
    }
}

/*
 * WKV-4 forward with a carried state and the receptance gate (RWKV-LLM page, "Time-mixing
 * block": eq. (14), and eq. (15)'s sigma(r_t) (.) wkv_t).  The state before the first token
 * of the call is (a, b, p): the past sums A = a e^p and B = b e^p of eq. (14) over every
 * token already consumed (NULL: empty).  Then, for t = 0 .. T-1,
 *     y_t = sigma(r_t) (A_t + e^{u+k_t} v_t) / (B_t + e^{u+k_t})     (sigma = 1 without r),
 *     A_{t+1} = e^{-w} A_t + e^{k_t} v_t,  B_{t+1} likewise,
 * and s_out receives (A_T, B_T) as (a, b, p) in double.  r is (B,T,C) float32 or NULL;
 * s_in is (B,C,3) float32 or NULL; s_out is (B,C,3) double or NULL.  A state with
 * a = b = 0 is empty whatever its p.
 */
void oracle_wkv4_forward_ex(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                            const float *k, const float *v, const float *r, const float *s_in,
                            double *y, double *s_out)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t bc = 0; bc < B * C; ++bc) {
        const int64_t b = bc / C, c = bc % C;
        const int64_t base = b * T * C + c;
        const double a0 = s_in ? (double)s_in[3 * bc] : 0.0;
        const double b0 = s_in ? (double)s_in[3 * bc + 1] : 0.0;
        const double p0 = s_in ? (double)s_in[3 * bc + 2] : 0.0;
        const int has_state = (a0 != 0.0 || b0 != 0.0);
        /* Common rescaling: e^{-K} for every weight, K the largest exponent present. */
        double K = T > 0 ? chan_max_k(k, T, C, base) : (has_state ? p0 : 0.0);
        if (has_state && p0 > K) K = p0;
        const double decay = exp(-(double)w[c]);
        const double uu = (double)u[c];
        double A = has_state ? a0 * exp(p0 - K) : 0.0;
        double Bs = has_state ? b0 * exp(p0 - K) : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const int64_t o = base + t * C;
            const double kt = (double)k[o], vt = (double)v[o];
            const double cur = exp(uu + kt - K);
            const double gate = r ? 1.0 / (1.0 + exp(-(double)r[o])) : 1.0;
            y[o] = gate * (A + cur * vt) / (Bs + cur);
            const double past = exp(kt - K);
            A = decay * A + past * vt;
            Bs = decay * Bs + past;
        }
        if (s_out) {
            s_out[3 * bc] = A;
            s_out[3 * bc + 1] = Bs;
            s_out[3 * bc + 2] = K;
        }
    }
}

/*
 * WKV-4 backward: gradients of a scalar loss L with upstream dL/dy = gy, w.r.t. the
 * w and u of eq. (14) as printed (summed over batch and time, since both are
 * per-channel vectors in that section) and w.r.t. every k_t and v_t.  The pages give
 * no backward; this is the chain rule applied to eq. (14).  With
 *   eps = e^{-w}, alpha_i = e^{k_i}, beta_t = e^{u+k_t},
 *   A_t = sum_{i<t} eps^{t-1-i} alpha_i v_i,   B_t = sum_{i<t} eps^{t-1-i} alpha_i,
 *   A'_t = sum_{i<t} (t-1-i) eps^{t-1-i} alpha_i v_i,  B'_t likewise without v,
 *   D_t = B_t + beta_t,  y_t = (A_t + beta_t v_t) / D_t,
 *   G_s = sum_{t>s} eps^{t-1-s} gy_t / D_t,   H_s = sum_{t>s} eps^{t-1-s} gy_t y_t / D_t:
 *
 *   dL/du   = sum_t gy_t beta_t (v_t - y_t) / D_t
 *   dL/dw   = - sum_t gy_t (A'_t - y_t B'_t) / D_t
 *   dL/dv_s = gy_s beta_s / D_s + alpha_s G_s
 *   dL/dk_s = gy_s beta_s (v_s - y_s) / D_s + alpha_s (v_s G_s - H_s)
 *
 * A' and B' follow A'_{t+1} = eps (A'_t + A_t); G and H run backwards with
 * G_{s-1} = gy_s / D_s + eps G_s from G_{T-1} = 0.
 * gw and gu are (C,); gk and gv are (B,T,C).
 */
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* r NULL: the plain operator.  Otherwise the output is sigma(r_t) y_t (eq. (15)); the sums
 * above then run with g_t = gy_t sigma(r_t), and gr_t = gy_t y_t sigma(r_t) (1 - sigma(r_t)).
 *
 * s_in (B,C,3) (a, b, p) or NULL: a carried state, A_0 = a e^p and B_0 = b e^p, decayed with
 * the sums (A_t = eps^t A_0 + ..., so A'_t gains t eps^t A_0 and dL/dw its share).
 * gs_out (B,C,2) or NULL: dL/d(a', b') of the state after the last token, s_out = (a', b', p')
 * with p' = s_out[.,.,2] held fixed, so dL/dA_T = a'-gradient e^{-p'}: it enters the reverse
 * sums as G_{T-1} = dL/dA_T, H_{T-1} = -dL/dB_T, and dL/dw gains -(dL/dA_T A'_T + dL/dB_T B'_T).
 * gs_in (B,C,2) or NULL: dL/d(a, b) of s_in with its p held fixed (p = 0 without s_in):
 * G_{-1} e^p and -H_{-1} e^p. */
static void wkv4_backward_impl(int64_t B, int64_t T, int64_t C,
                               const float *w, const float *u,
                               const float *k, const float *v, const float *r, const float *gy,
                               double *gw, double *gu, double *gk, double *gv, double *gr,
                               const float *s_in, const float *s_out, const float *gs_out, double *gs_in,
                               double *cw, double *cu)
{
    double *gw_bc = (double *)calloc((size_t)(B * C), sizeof(double));
    double *gu_bc = (double *)calloc((size_t)(B * C), sizeof(double));
    double *cw_bc = (double *)calloc((size_t)(B * C), sizeof(double));
    double *cu_bc = (double *)calloc((size_t)(B * C), sizeof(double));
#pragma omp parallel
    {
        double *D = (double *)malloc((size_t)T * sizeof(double));
        double *Y = (double *)malloc((size_t)T * sizeof(double));
#pragma omp for schedule(dynamic, 4)
        for (int64_t bc = 0; bc < B * C; ++bc) {
            const int64_t b = bc / C, c = bc % C;
            const int64_t base = b * T * C + c;
            const double p0 = s_in ? (double)s_in[3 * bc + 2] : 0.0;
            if (T == 0) {
                /* No tokens: the state passes through, s_out = s_in. */
                gw_bc[bc] = gu_bc[bc] = 0.0;
                if (gs_in) {
                    const double f = gs_out ? exp(p0 - (double)s_out[3 * bc + 2]) : 0.0;
                    gs_in[2 * bc] = gs_out ? (double)gs_out[2 * bc] * f : 0.0;
                    gs_in[2 * bc + 1] = gs_out ? (double)gs_out[2 * bc + 1] * f : 0.0;
                }
                continue;
            }
            double K = chan_max_k(k, T, C, base);
            if (s_in && (s_in[3 * bc] != 0.0f || s_in[3 * bc + 1] != 0.0f) && p0 > K) K = p0;
            const double eps = exp(-(double)w[c]);
            const double uu = (double)u[c];
            double A = s_in ? (double)s_in[3 * bc] * exp(p0 - K) : 0.0;
            double Bs = s_in ? (double)s_in[3 * bc + 1] * exp(p0 - K) : 0.0;
            double Ad = 0.0, Bd = 0.0, sgw = 0.0, sgu = 0.0;
            /* Magnitude sums (cw, cu): A and A' with |v| in place of v. */
            double Aabs = s_in ? fabs((double)s_in[3 * bc]) * exp(p0 - K) : 0.0, Adabs = 0.0, cgw = 0.0, cgu = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                const int64_t o = base + t * C;
                const double kt = (double)k[o], vt = (double)v[o];
                const double g = r ? (double)gy[o] * sigmoid((double)r[o]) : (double)gy[o];
                const double beta = exp(uu + kt - K);
                const double alpha = exp(kt - K);
                const double Dt = Bs + beta;
                const double yt = (A + beta * vt) / Dt;
                D[t] = Dt;
                Y[t] = yt;
                if (gr) {
                    const double sg = sigmoid((double)r[o]);
                    gr[o] = (double)gy[o] * yt * sg * (1.0 - sg);
                }
                sgu += g * beta * (vt - yt) / Dt;
                sgw -= g * (Ad - yt * Bd) / Dt;
                cgu += fabs(g) * beta * (fabs(vt) + fabs(yt)) / Dt;
                cgw += fabs(g) * (Adabs + fabs(yt) * Bd) / Dt;
                Adabs = eps * (Adabs + Aabs);
                Aabs = eps * Aabs + alpha * fabs(vt);
                Ad = eps * (Ad + A);
                Bd = eps * (Bd + Bs);
                A = eps * A + alpha * vt;
                Bs = eps * Bs + alpha;
            }
            /* The state after the last token: its gradient seeds the reverse sums. */
            const double so = gs_out ? exp(K - (double)s_out[3 * bc + 2]) : 0.0;
            const double gA = gs_out ? (double)gs_out[2 * bc] * so : 0.0;   /* dL/dA_T e^K */
            const double gB = gs_out ? (double)gs_out[2 * bc + 1] * so : 0.0;
            sgw -= gA * Ad + gB * Bd;
            cgw += fabs(gA) * Adabs + fabs(gB) * Bd;
            gw_bc[bc] = sgw;
            gu_bc[bc] = sgu;
            cw_bc[bc] = cgw;
            cu_bc[bc] = cgu;
            double G = gA, H = -gB; /* G_{T-1}, H_{T-1} */
            for (int64_t s = T - 1; s >= 0; --s) {
                const int64_t o = base + s * C;
                const double ks = (double)k[o], vs = (double)v[o];
                const double g = r ? (double)gy[o] * sigmoid((double)r[o]) : (double)gy[o];
                const double beta = exp(uu + ks - K);
                const double alpha = exp(ks - K);
                const double q = g / D[s];
                gv[o] = q * beta + alpha * G;
                gk[o] = q * beta * (vs - Y[s]) + alpha * (vs * G - H);
                G = q + eps * G;      /* becomes G_{s-1} */
                H = q * Y[s] + eps * H;
            }
            if (gs_in) {
                gs_in[2 * bc] = G * exp(p0 - K);
                gs_in[2 * bc + 1] = -H * exp(p0 - K);
            }
        }
        free(D);
        free(Y);
    }
    for (int64_t c = 0; c < C; ++c) {
        double sw = 0.0, su = 0.0;
        for (int64_t b = 0; b < B; ++b) {
            sw += gw_bc[b * C + c];
            su += gu_bc[b * C + c];
        }
        gw[c] = sw;
        gu[c] = su;
        if (cw) {
            double a = 0.0, b2 = 0.0;
            for (int64_t b = 0; b < B; ++b) {
                a += cw_bc[b * C + c];
                b2 += cu_bc[b * C + c];
            }
            cw[c] = a;
            cu[c] = b2;
        }
    }
    free(gw_bc);
    free(gu_bc);
    free(cw_bc);
    free(cu_bc);
}

void oracle_wkv4_backward(int64_t B, int64_t T, int64_t C,
                          const float *w, const float *u,
                          const float *k, const float *v, const float *gy,
                          double *gw, double *gu, double *gk, double *gv)
{
    wkv4_backward_impl(B, T, C, w, u, k, v, NULL, gy, gw, gu, gk, gv, NULL, NULL, NULL, NULL, NULL, NULL, NULL);
}

/*
 * Backward of the gated output o_t = sigma(r_t) wkv_t (RWKV-LLM page, eq. (15), before W_o)
 * given gy = dL/do: the WKV gradients with dL/dwkv_t = gy_t sigma(r_t), and
 * gr_t = dL/dr_t = gy_t wkv_t sigma(r_t) (1 - sigma(r_t)).  gr is (B,T,C) double.
 */
void oracle_wkv4_backward_gated(int64_t B, int64_t T, int64_t C,
                                const float *w, const float *u, const float *k, const float *v,
                                const float *r, const float *gy,
                                double *gw, double *gu, double *gk, double *gv, double *gr)
{
    wkv4_backward_impl(B, T, C, w, u, k, v, r, gy, gw, gu, gk, gv, gr, NULL, NULL, NULL, NULL, NULL, NULL);
}

/*
 * Backward with a carried state (the forward is oracle_wkv4_forward_ex): r and gr as in
 * oracle_wkv4_backward_gated (NULL for the plain output); s_in, s_out, gs_out, gs_in as
 * described at wkv4_backward_impl.  Any of them may be NULL.
 */
void oracle_wkv4_backward_ex(int64_t B, int64_t T, int64_t C, const float *w, const float *u, const float *k,
                             const float *v, const float *r, const float *s_in, const float *s_out,
                             const float *gy, const float *gs_out, double *gw, double *gu, double *gk, double *gv,
                             double *gr, double *gs_in)
{
    wkv4_backward_impl(B, T, C, w, u, k, v, r, gy, gw, gu, gk, gv, gr, s_in, s_out, gs_out, gs_in, NULL, NULL);
}

/*
 * As oracle_wkv4_backward_ex, also returning per channel the sums over b and t of the
 * magnitudes of the products that make up each term of dL/dw and dL/du (test
 * infrastructure: the conditioning of those sums, for their per-channel tolerance):
 *   cu[c] = sum_{b,t} |g_t| beta_t (|v_t| + |y_t|) / D_t
 *   cw[c] = sum_{b,t} |g_t| (|A'|_t + |y_t| B'_t) / D_t  + |dL/dA_T| |A'|_T + |dL/dB_T| B'_T
 * with |A'| the sum A' taken over |v_i|.  An evaluation that rounds every product and
 * partial sum to float32 is off by a few float32 ulps of these, whatever the sums cancel to.
 */
void oracle_wkv4_backward_cond(int64_t B, int64_t T, int64_t C, const float *w, const float *u, const float *k,
                               const float *v, const float *r, const float *s_in, const float *s_out,
                               const float *gy, const float *gs_out, double *gw, double *gu, double *gk, double *gv,
                               double *gr, double *gs_in, double *cw, double *cu)
{
    wkv4_backward_impl(B, T, C, w, u, k, v, r, gy, gw, gu, gk, gv, gr, s_in, s_out, gs_out, gs_in, cw, cu);
}

/*
 * Real diagonal scan x_t = a_t x_{t-1} + b_t, the scan form the minGRU page gives as
 * the target of a parallel scan ("Were RNNs All We Needed?" news page, minGRU
 * section: v_t = a_t (.) v_{t-1} + b_t).  x_{-1} = x0[b,c], or 0 when x0 is NULL.
 */
void oracle_scan_real(int64_t B, int64_t T, int64_t C,
                      const float *a, const float *bb, const float *x0, double *x)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t bc = 0; bc < B * C; ++bc) {
        const int64_t b = bc / C, c = bc % C;
        const int64_t base = b * T * C + c;
        double s = x0 ? (double)x0[b * C + c] : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const int64_t o = base + t * C;
            s = (double)a[o] * s + (double)bb[o];
            x[o] = s;
        }
    }
}

/*
 * Complex diagonal scan x_t = lambda x_{t-1} + u_t, the LRU write-up's element-wise
 * complex recurrence (section on the diagonal linear RNN, eq. lr-xx), in complex128.
 * lambda is (C,) complex64, u is (B,T,C) complex64, x0 is (B,C) complex64 or NULL
 * (zero, which gives x_0 = u_0 as in the write-up's unrolled form, eq. lr-e).
 * x is (B,T,C) complex128, interleaved.
 */
void oracle_scan_complex(int64_t B, int64_t T, int64_t C,
                         const float *lam, const float *u, const float *x0, double *x)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t bc = 0; bc < B * C; ++bc) {
        const int64_t b = bc / C, c = bc % C;
        const int64_t base = b * T * C + c;
        const double complex L = (double)lam[2 * c] + (double)lam[2 * c + 1] * I;
        double complex s = 0.0;
        if (x0) s = (double)x0[2 * (b * C + c)] + (double)x0[2 * (b * C + c) + 1] * I;
        for (int64_t t = 0; t < T; ++t) {
            const int64_t o = base + t * C;
            const double complex ut = (double)u[2 * o] + (double)u[2 * o + 1] * I;
            s = L * s + ut;
            x[2 * o] = creal(s);
            x[2 * o + 1] = cimag(s);
        }
    }
}

/*
 * Backward of the real diagonal scan x_t = a_t x_{t-1} + b_t (minGRU page, scan form;
 * the pages give no backward).  For upstream gradients gx_t = dL/dx_t, the adjoint runs
 * backwards in time:
 *     gb_t = gx_t + a_{t+1} gb_{t+1}   (gb_{T-1} = gx_{T-1}),
 *     ga_t = gb_t x_{t-1}              (x_{-1} = x0, or 0 without x0),
 *     gx0  = a_0 gb_0                  (the initial state's gradient, also for a zero x0).
 * x is the forward output (B,T,C) in double; a, gx are (B,T,C) float32; x0 is (B,C) or
 * NULL.  Outputs ga, gb (B,T,C) and gx0 (B,C, may be NULL) in double.
 */
void oracle_scan_real_backward(int64_t B, int64_t T, int64_t C, const float *a, const float *x0,
                               const double *x, const float *gx, double *ga, double *gb,
                               double *gx0)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t bc = 0; bc < B * C; ++bc) {
        const int64_t b = bc / C, c = bc % C;
        const int64_t base = b * T * C + c;
        double s = 0.0;  /* gb_{t+1} */
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t o = base + t * C;
            const double anext = (t + 1 < T) ? (double)a[o + C] : 0.0;
            s = (double)gx[o] + anext * s;
            gb[o] = s;
            const double xprev = (t > 0) ? x[o - C] : (x0 ? (double)x0[b * C + c] : 0.0);
            ga[o] = s * xprev;
        }
        if (gx0) gx0[b * C + c] = (T > 0) ? (double)a[base] * s : 0.0;
    }
}

/*
 * Backward of the complex diagonal scan x_t = lambda x_{t-1} + u_t (LRU write-up, eq.
 * lr-xx; the pages give no backward).  Gradients of a real loss are taken as
 * dL/dRe + i dL/dIm, so that dL = Re sum conj(g) dz.  Backwards in time:
 *     gu_t = gx_t + conj(lambda) gu_{t+1},
 *     glambda = sum over batch and time of gu_t conj(x_{t-1})   (x_{-1} = x0 or 0),
 *     gx0 = conj(lambda) gu_0                                   (also for a zero x0).
 * lambda (C,) and gx (B,T,C) are complex64, x0 (B,C) complex64 or NULL, x (B,T,C)
 * complex128; outputs glambda (C,), gu (B,T,C), gx0 (B,C, may be NULL) complex128.
 * glambda adds the batch rows in ascending order.
 */
void oracle_scan_complex_backward(int64_t B, int64_t T, int64_t C, const float *lam, const float *x0,
                                  const double *x, const float *gx, double *glam, double *gu,
                                  double *gx0)
{
    double *part = (double *)calloc((size_t)(B * C) * 2 + 1, sizeof(double));
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t bc = 0; bc < B * C; ++bc) {
        const int64_t b = bc / C, c = bc % C;
        const int64_t base = b * T * C + c;
        const double complex Lc = conj((double)lam[2 * c] + (double)lam[2 * c + 1] * I);
        const double complex z0 = x0 ? (double)x0[2 * (b * C + c)] + (double)x0[2 * (b * C + c) + 1] * I : 0.0;
        double complex s = 0.0, acc = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t o = base + t * C;
            s = ((double)gx[2 * o] + (double)gx[2 * o + 1] * I) + Lc * s;
            gu[2 * o] = creal(s);
            gu[2 * o + 1] = cimag(s);
            const double complex xp = (t > 0) ? x[2 * (o - C)] + x[2 * (o - C) + 1] * I : z0;
            acc += s * conj(xp);
        }
        part[2 * bc] = creal(acc);
        part[2 * bc + 1] = cimag(acc);
        if (gx0) {
            const double complex g0 = (T > 0) ? Lc * s : 0.0;
            gx0[2 * (b * C + c)] = creal(g0);
            gx0[2 * (b * C + c) + 1] = cimag(g0);
        }
    }
    for (int64_t c = 0; c < C; ++c) {
        double re = 0.0, im = 0.0;
        for (int64_t b = 0; b < B; ++b) {
            re += part[2 * (b * C + c)];
            im += part[2 * (b * C + c) + 1];
        }
        glam[2 * c] = re;
        glam[2 * c + 1] = im;
    }
    free(part);
}

/*
 * Token shift of the RWKV time-mix block.  RWKV-LLM page, section "Time-mixing block",
 * eqs. (11)-(13): each projection input is a per-channel linear interpolation between
 * the current token and the previous one (the page calls the recurrent form a linear
 * interpolation of the current and previous inputs),
 *
 *   xm[m,b,t,c] = mu[m,c] x[b,t,c] + (1 - mu[m,c]) x[b,t-1,c],   m = 0 .. M-1,
 *
 * with x[b,-1,c] = x_prev[b,c] (the last token of an earlier call) or 0.  x (B,T,C),
 * x_prev (B,C) or NULL, mu (M,C) float32; out (M,B,T,C) float64.
 */
void oracle_token_shift(int64_t B, int64_t T, int64_t C, int64_t M, const float *x, const float *x_prev,
                        const float *mu, double *out)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t bc = 0; bc < B * C; ++bc) {
        const int64_t b = bc / C, c = bc % C;
        const int64_t base = b * T * C + c;
        for (int64_t m = 0; m < M; ++m) {
            const double mm = (double)mu[m * C + c];
            double prev = x_prev ? (double)x_prev[b * C + c] : 0.0;
            for (int64_t t = 0; t < T; ++t) {
                const double cur = (double)x[base + t * C];
                out[m * B * T * C + base + t * C] = mm * cur + (1.0 - mm) * prev;
                prev = cur;
            }
        }
    }
}

/*
 * Backward of oracle_token_shift (the pages give none; chain rule of eqs. (11)-(13)).
 * With g = dL/dxm (M,B,T,C):
 *   gx[b,t,c]     = sum_m ( mu[m,c] g[m,b,t,c] + (1 - mu[m,c]) g[m,b,t+1,c] )   (no t+1 term at T-1)
 *   gx_prev[b,c]  = sum_m (1 - mu[m,c]) g[m,b,0,c]
 *   gmu[m,c]      = sum over b and t of g[m,b,t,c] (x[b,t,c] - x[b,t-1,c])
 * gmu adds each row's time sum, then the batch rows in ascending order.  gx (B,T,C),
 * gmu (M,C) and gx_prev (B,C, may be NULL) are float64.
 */
void oracle_token_shift_backward(int64_t B, int64_t T, int64_t C, int64_t M, const float *x,
                                 const float *x_prev, const float *mu, const float *g, double *gx,
                                 double *gmu, double *gx_prev)
{
    double *part = (double *)calloc((size_t)(M * B * C) + 1, sizeof(double));
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t bc = 0; bc < B * C; ++bc) {
        const int64_t b = bc / C, c = bc % C;
        const int64_t base = b * T * C + c;
        for (int64_t t = 0; t < T; ++t) gx[base + t * C] = 0.0;
        double gp = 0.0;
        for (int64_t m = 0; m < M; ++m) {
            const double mm = (double)mu[m * C + c];
            const float *gm = g + m * B * T * C;
            double acc = 0.0;
            double prev = x_prev ? (double)x_prev[b * C + c] : 0.0;
            for (int64_t t = 0; t < T; ++t) {
                const int64_t o = base + t * C;
                const double gt = (double)gm[o];
                const double gnext = (t + 1 < T) ? (double)gm[o + C] : 0.0;
                gx[o] += mm * gt + (1.0 - mm) * gnext;
                const double cur = (double)x[o];
                acc += gt * (cur - prev);
                prev = cur;
            }
            part[m * B * C + bc] = acc;
            if (T > 0) gp += (1.0 - mm) * (double)gm[base];
        }
        if (gx_prev) gx_prev[b * C + c] = gp;
    }
    for (int64_t m = 0; m < M; ++m)
        for (int64_t c = 0; c < C; ++c) {
            double s = 0.0;
            for (int64_t b = 0; b < B; ++b) s += part[m * B * C + b * C + c];
            gmu[m * C + c] = s;
        }
    free(part);
}

/*
 * minGRU in scan form (minGRU page: the GRU reduced to v_t = a_t (.) v_{t-1} + b_t once the
 * hidden-state dependence and the tanh are dropped; the page's equations are images, and
 * the reading is h_t = (1 - z_t) h_{t-1} + z_t h~_t with z_t = sigmoid of the gate's
 * pre-activation).  kz (B,T,C) pre-activations, h (B,T,C) candidates h~, x0 (B,C) or NULL
 * (zero); x (B,T,C) double.
 */
void oracle_scan_mingru(int64_t B, int64_t T, int64_t C, const float *kz, const float *h, const float *x0,
                        double *x)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t bc = 0; bc < B * C; ++bc) {
        const int64_t b = bc / C, c = bc % C;
        const int64_t base = b * T * C + c;
        double s = x0 ? (double)x0[b * C + c] : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const int64_t o = base + t * C;
            const double z = 1.0 / (1.0 + exp(-(double)kz[o]));
            s = (1.0 - z) * s + z * (double)h[o];
            x[o] = s;
        }
    }
}

/*
 * minLSTM in scan form (minGRU page, minLSTM section: the output gate and the cell are
 * dropped and the two remaining gates are normalised to share the hidden state's input):
 * f_t = sigmoid(kf_t), i_t = sigmoid(ki_t), f'_t = f_t / (f_t + i_t), i'_t = i_t / (f_t + i_t),
 * h_t = f'_t h_{t-1} + i'_t h~_t.  Valid while sigmoid(kf) + sigmoid(ki) does not
 * underflow double (logits above about -700).
 */
void oracle_scan_minlstm(int64_t B, int64_t T, int64_t C, const float *kf, const float *ki, const float *h,
                         const float *x0, double *x)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t bc = 0; bc < B * C; ++bc) {
        const int64_t b = bc / C, c = bc % C;
        const int64_t base = b * T * C + c;
        double s = x0 ? (double)x0[b * C + c] : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const int64_t o = base + t * C;
            const double f = 1.0 / (1.0 + exp(-(double)kf[o]));
            const double i = 1.0 / (1.0 + exp(-(double)ki[o]));
            s = (f / (f + i)) * s + (i / (f + i)) * (double)h[o];
            x[o] = s;
        }
    }
}

/*
 * Real scan with one decay per channel (an SLRU, the LRU write-up's section on RWKV: each of
 * RWKV's two sums is such a recurrence): x_t = lambda_c x_{t-1} + u_t.  lambda (C), u
 * (B,T,C), x0 (B,C) or NULL; x (B,T,C) double.
 */
void oracle_scan_real_decay(int64_t B, int64_t T, int64_t C, const float *lam, const float *u, const float *x0,
                            double *x)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t bc = 0; bc < B * C; ++bc) {
        const int64_t b = bc / C, c = bc % C;
        const int64_t base = b * T * C + c;
        const double L = (double)lam[c];
        double s = x0 ? (double)x0[b * C + c] : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const int64_t o = base + t * C;
            s = L * s + (double)u[o];
            x[o] = s;
        }
    }
}

/*
 * gamma = sqrt(1 - |lambda|^2), the normalised LRU's input scale, for a lambda of modulus
 * r in [0, 1] (LRU write-up: the polar form with r in [0, 1]; the initialisation section's
 * state variance 1 / (1 - r^2)).  A unit-modulus lambda stored as complex64 often has
 * |lambda|^2 a rounding above 1; it takes the value at r = 1, gamma = 0.
 */
static double lru_gamma(double complex L)
{
    return sqrt(fmax(0.0, 1.0 - creal(L * conj(L))));
}

/*
 * The LRU's normalised input (LRU write-up, initialisation section: with |lambda| < 1 a
 * stationary input of variance s feeds a state of variance s / (1 - |lambda|^2), so the
 * input is scaled by gamma = sqrt(1 - |lambda|^2) to keep the state's scale):
 * x_t = lambda x_{t-1} + gamma u_t, gamma per channel (lru_gamma).  Arguments as
 * oracle_scan_complex.
 */
void oracle_scan_complex_normalized(int64_t B, int64_t T, int64_t C, const float *lam, const float *u,
                                    const float *x0, double *x)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t bc = 0; bc < B * C; ++bc) {
        const int64_t b = bc / C, c = bc % C;
        const int64_t base = b * T * C + c;
        const double complex L = (double)lam[2 * c] + (double)lam[2 * c + 1] * I;
        const double gamma = lru_gamma(L);
        double complex s = 0.0;
        if (x0) s = (double)x0[2 * (b * C + c)] + (double)x0[2 * (b * C + c) + 1] * I;
        for (int64_t t = 0; t < T; ++t) {
            const int64_t o = base + t * C;
            const double complex ut = (double)u[2 * o] + (double)u[2 * o + 1] * I;
            s = L * s + gamma * ut;
            x[2 * o] = creal(s);
            x[2 * o + 1] = cimag(s);
        }
    }
}

/*
 * Backward of minGRU (the pages give none; chain rule of the minGRU reading above).  With
 * z_t = sigmoid(kz_t) and d_t = dL/dh_t, the total gradient of the hidden state,
 *     d_t = gx_t + (1 - z_{t+1}) d_{t+1}          (d_T = 0)
 *     dL/dz_t  = d_t (h~_t - h_{t-1}),   dL/dkz_t = dL/dz_t z_t (1 - z_t)
 *     dL/dh~_t = d_t z_t,                dL/dx0   = (1 - z_0) d_0
 * x is the forward output (double), h_{-1} = x0 or 0.  gx0 may be NULL.
 */
void oracle_scan_mingru_backward(int64_t B, int64_t T, int64_t C, const float *kz, const float *h,
                                 const float *x0, const double *x, const float *gx, double *gkz,
                                 double *gh, double *gx0)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t bc = 0; bc < B * C; ++bc) {
        const int64_t b = bc / C, c = bc % C;
        const int64_t base = b * T * C + c;
        const double h0 = x0 ? (double)x0[b * C + c] : 0.0;
        double d = 0.0, znext = 0.0;  /* d_{t+1} and z_{t+1}; the step after the last adds nothing */
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t o = base + t * C;
            const double z = 1.0 / (1.0 + exp(-(double)kz[o]));
            d = (double)gx[o] + (t + 1 < T ? (1.0 - znext) * d : 0.0);
            const double hprev = t > 0 ? x[o - C] : h0;
            gkz[o] = d * ((double)h[o] - hprev) * z * (1.0 - z);
            gh[o] = d * z;
            znext = z;
        }
        if (gx0) gx0[b * C + c] = T > 0 ? (1.0 - znext) * d : 0.0;
    }
}

/*
 * Backward of minLSTM (chain rule of the minLSTM reading above).  With f = sigmoid(kf),
 * i = sigmoid(ki), a = f / (f + i) (the weight of h_{t-1}; i / (f + i) = 1 - a weighs h~):
 *     d_t = gx_t + a_{t+1} d_{t+1},   dL/da_t = d_t (h_{t-1} - h~_t),   dL/dh~_t = d_t (1 - a_t)
 *     da/df = i / (f + i)^2,  da/di = -f / (f + i)^2,  df/dkf = f (1 - f),  di/dki = i (1 - i)
 *     dL/dx0 = a_0 d_0
 */
void oracle_scan_minlstm_backward(int64_t B, int64_t T, int64_t C, const float *kf, const float *ki,
                                  const float *h, const float *x0, const double *x, const float *gx,
                                  double *gkf, double *gki, double *gh, double *gx0)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t bc = 0; bc < B * C; ++bc) {
        const int64_t b = bc / C, c = bc % C;
        const int64_t base = b * T * C + c;
        const double h0 = x0 ? (double)x0[b * C + c] : 0.0;
        double d = 0.0, anext = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t o = base + t * C;
            const double f = 1.0 / (1.0 + exp(-(double)kf[o]));
            const double i = 1.0 / (1.0 + exp(-(double)ki[o]));
            const double a = f / (f + i);
            d = (double)gx[o] + (t + 1 < T ? anext * d : 0.0);
            const double hprev = t > 0 ? x[o - C] : h0;
            const double ga = d * (hprev - (double)h[o]);
            gkf[o] = ga * i / ((f + i) * (f + i)) * f * (1.0 - f);
            gki[o] = -ga * f / ((f + i) * (f + i)) * i * (1.0 - i);
            gh[o] = d * (1.0 - a);
            anext = a;
        }
        if (gx0) gx0[b * C + c] = T > 0 ? anext * d : 0.0;
    }
}

/*
 * Backward of the real scan with one decay per channel, x_t = lam_c x_{t-1} + u_t:
 *     gu_t = gx_t + lam_c gu_{t+1},   glam_c = sum over batch and time of gu_t x_{t-1},
 *     gx0 = lam_c gu_0.   glam adds the batch rows in ascending order.
 */
void oracle_scan_real_decay_backward(int64_t B, int64_t T, int64_t C, const float *lam, const float *x0,
                                     const double *x, const float *gx, double *glam, double *gu, double *gx0)
{
    double *part = (double *)calloc((size_t)(B * C) + 1, sizeof(double));
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t bc = 0; bc < B * C; ++bc) {
        const int64_t b = bc / C, c = bc % C;
        const int64_t base = b * T * C + c;
        const double L = (double)lam[c];
        const double h0 = x0 ? (double)x0[b * C + c] : 0.0;
        double s = 0.0, acc = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t o = base + t * C;
            s = (double)gx[o] + L * s;
            gu[o] = s;
            acc += s * (t > 0 ? x[o - C] : h0);
        }
        part[bc] = acc;
        if (gx0) gx0[b * C + c] = T > 0 ? L * s : 0.0;
    }
    for (int64_t c = 0; c < C; ++c) {
        double sum = 0.0;
        for (int64_t b = 0; b < B; ++b) sum += part[b * C + c];
        glam[c] = sum;
    }
    free(part);
}

/*
 * Backward of the LRU with normalised input, x_t = lambda x_{t-1} + gamma u_t with
 * gamma = sqrt(1 - |lambda|^2) (gradients as dL/dRe + i dL/dIm, as for the complex scan):
 *     s_t = gx_t + conj(lambda) s_{t+1},   dL/du_t = gamma s_t,   dL/dx0 = conj(lambda) s_0,
 *     dL/dgamma = sum over batch and time of Re(conj(s_t) u_t),
 *     glambda = sum of s_t conj(x_{t-1}) + dL/dgamma (dgamma/dRe + i dgamma/dIm)
 *             = sum of s_t conj(x_{t-1}) - (dL/dgamma / gamma) lambda,
 * the last term taken as 0 where gamma = 0 (|lambda| = 1, where gamma has no derivative).
 */
void oracle_scan_complex_normalized_backward(int64_t B, int64_t T, int64_t C, const float *lam, const float *u,
                                             const float *x0, const double *x, const float *gx, double *glam,
                                             double *gu, double *gx0)
{
    double *part = (double *)calloc((size_t)(B * C) * 3 + 1, sizeof(double));
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t bc = 0; bc < B * C; ++bc) {
        const int64_t b = bc / C, c = bc % C;
        const int64_t base = b * T * C + c;
        const double complex L = (double)lam[2 * c] + (double)lam[2 * c + 1] * I;
        const double gamma = lru_gamma(L);
        const double complex z0 = x0 ? (double)x0[2 * (b * C + c)] + (double)x0[2 * (b * C + c) + 1] * I : 0.0;
        double complex s = 0.0, acc = 0.0;
        double dgam = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t o = base + t * C;
            s = ((double)gx[2 * o] + (double)gx[2 * o + 1] * I) + conj(L) * s;
            gu[2 * o] = gamma * creal(s);
            gu[2 * o + 1] = gamma * cimag(s);
            const double complex xp = t > 0 ? x[2 * (o - C)] + x[2 * (o - C) + 1] * I : z0;
            acc += s * conj(xp);
            const double complex ut = (double)u[2 * o] + (double)u[2 * o + 1] * I;
            dgam += creal(conj(s) * ut);
        }
        part[3 * bc] = creal(acc);
        part[3 * bc + 1] = cimag(acc);
        part[3 * bc + 2] = dgam;
        if (gx0) {
            const double complex g0 = T > 0 ? conj(L) * s : 0.0;
            gx0[2 * (b * C + c)] = creal(g0);
            gx0[2 * (b * C + c) + 1] = cimag(g0);
        }
    }
    for (int64_t c = 0; c < C; ++c) {
        const double complex L = (double)lam[2 * c] + (double)lam[2 * c + 1] * I;
        const double gamma = lru_gamma(L);
        double re = 0.0, im = 0.0, dg = 0.0;
        for (int64_t b = 0; b < B; ++b) {
            re += part[3 * (b * C + c)];
            im += part[3 * (b * C + c) + 1];
            dg += part[3 * (b * C + c) + 2];
        }
        const double k = gamma > 0.0 ? dg / gamma : 0.0;
        glam[2 * c] = re - k * creal(L);
        glam[2 * c + 1] = im - k * cimag(L);
    }
    free(part);
}

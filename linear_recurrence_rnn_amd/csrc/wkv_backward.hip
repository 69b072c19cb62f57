// wkv_backward.hip -- WKV-4 backward on gfx950.
//
// Chain rule of eq. (14) of the RWKV-LLM page ("Time-mixing block"); the pages give no
// backward.  With eps = e^{-w}, alpha_i = e^{k_i}, beta_t = e^{u+k_t}, D_t = B_t + beta_t,
//   dL/du   = sum_t g_t beta_t (v_t - y_t) / D_t
//   dL/dw   = -sum_t g_t (A'_t - y_t B'_t) / D_t,   A'_t = sum_{i<t} (t-1-i) eps^{t-1-i} alpha_i v_i
//   dL/dv_s = g_s beta_s / D_s + alpha_s G_s,       G_s = sum_{t>s} eps^{t-1-s} g_t / D_t
//   dL/dk_s = g_s beta_s (v_s - y_s) / D_s + alpha_s (v_s G_s - H_s),  H_s likewise with g_t y_t
// v_t - y_t is formed as 2^{p-q} (v_t b - a) / dm (no cancellation, exactly 0 at t = 0).
//
// Two streaming kernels, laid out like the forward scan: a workgroup owns one slab of NW
// chunks of L steps of one channel group (64 lanes x VEC contiguous channels), wave w holds
// chunk w in registers, and every wave-wide access is one contiguous row segment.
//   state kernel     forward sums (A, B, A', B') of each chunk -> LDS scan over the slab ->
//                    decoupled look-back over the earlier slabs -> the sums at every slab
//                    end are published (the last slab has no successor and is skipped);
//   gradient kernel  slabs in reverse time order.  Re-run the forward from the previous
//                    slab's published sums (per step y, v - y, the exponent q and g/D; the
//                    dL/dw, dL/du terms), reduce the reverse sums (G, H) of each chunk, scan
//                    them over the slab, look back over the LATER slabs for the reverse
//                    carry, re-run the reverse and write dL/dk, dL/dv.  A slab's dL/dw, dL/du
//                    sums ride in its reverse look-back record, so the first slab of a
//                    sequence ends with the sums of the whole row;
//   a third kernel sums the rows over the batch in order.
// HBM traffic: k, v twice, g once, dL/dk, dL/dv once (28 bytes per element; 20 algorithmic).
//
// The sums are float64 mantissas times 2^p with p an integer exponent (wkv_math.hpp).  The
// gradients are differences of long sums (v G - H, A' - y B'): float64 mantissas keep their
// rounding from accumulating along the sequence; exponentials, reciprocals and the per-step
// values held in registers stay float32.  On this GPU a float64 FMA issues at the rate of an
// unpacked float32 FMA.
// Every sum over slabs is a fold in chain order (look-back), and dL/dw, dL/du are summed over
// the batch in ascending row order: the results do not depend on scheduling.
#include "device_common.hpp"
#include "lookback.hpp"
#include "wkv_backward.hpp"
#include "wkv_math.hpp"

namespace linrec {

namespace {

// Forward sums over a span: A = a 2^p, B = b 2^p, A' = ad 2^p, B' = bd 2^p.
struct Fwd { double a, b, ad, bd; float p; };
// Reverse sums: G-like = x 2^r, H-like = h 2^r; z 2^r is the sum of the (positive) weights,
// which x and h can cancel below, and sets the exponent.
struct Rev { double x, h, z; float r; };
// Reverse look-back record: the reverse sums of a run of slabs and their dL/dw, dL/du sums.
struct RevRec { Rev st; double sw, su; };

__device__ __forceinline__ Fwd fwd_identity() { return {0.0, 0.0, 0.0, 0.0, kEmpty}; }
__device__ __forceinline__ Rev rev_identity() { return {0.0, 0.0, 0.0, kEmpty}; }

// State s1, then a span s2 of n2 steps:
//   A = eps^n2 A1 + A2,   A' = eps^n2 (A'1 + n2 A1) + A'2   (B, B' likewise).
__device__ __forceinline__ Fwd fwd_combine(float om, const Fwd& s1, const Fwd& s2, int64_t n2) {
    float p, f1, f2;
    merge_scales(s1.p, (float)s1.b, s2.p, (float)s2.b, mul_split((float)n2, om), p, f1, f2);
    const double g1 = f1, g2 = f2, fn = (double)n2;
    return {fma(s1.a, g1, s2.a * g2), fma(s1.b, g1, s2.b * g2), fma(fma(fn, s1.a, s1.ad), g1, s2.ad * g2),
            fma(fma(fn, s1.b, s1.bd), g1, s2.bd * g2), p};
}

// Reverse sums: s1 is the state at the end of an earlier span s2 of n2 steps; the result is
// the state at the start of s2:  X = s2 + eps^n2 s1.
__device__ __forceinline__ Rev rev_combine(float om, const Rev& s1, const Rev& s2, int64_t n2) {
    float r, f1, f2;
    merge_scales(s1.r, (float)s1.z, s2.r, (float)s2.z, mul_split((float)n2, om), r, f1, f2);
    const double g1 = f1, g2 = f2;
    return {fma(s1.x, g1, s2.x * g2), fma(s1.h, g1, s2.h * g2), fma(s1.z, g1, s2.z * g2), r};
}

// (A, B, A', B') of a chunk of n steps from the empty state: with m_j = kk_j - (n-1-j) om,
// p = ceil(max m_j), weights 2^{m_j - p}; A' and B' weight step j by its distance n-1-j.
template <int L, int VEC>
__device__ __forceinline__ Fwd fwd_chunk(float om, const float (&kk)[L][VEC], const float (&vv)[L][VEC],
                                         int e, int n) {
    if (n <= 0) return fwd_identity();
    float m[L];
    float mx = kEmpty;
#pragma unroll
    for (int j = 0; j < L; ++j) {
        m[j] = (j < n) ? fmaf(-(float)(n - 1 - j), om, kk[j][e]) : kEmpty;
        mx = fmaxf(mx, m[j]);
    }
    Fwd s = fwd_identity();
    s.p = ceilf(mx);
#pragma unroll
    for (int j = 0; j < L; ++j) {
        const double f = fast_exp2(m[j] - s.p);  // 0 for the unused slots
        const double fd = f * (double)max(n - 1 - j, 0);
        s.a = fma(f, (double)vv[j][e], s.a);
        s.b += f;
        s.ad = fma(fd, (double)vv[j][e], s.ad);
        s.bd += fd;
    }
    return s;
}

// The forward sums advanced past one step (kj = k log2 e).
__device__ __forceinline__ void fwd_advance(float om, Fwd& s, float kj, double vj, float M) {
    const float q2 = ceilf(fmaxf(M - om, kj));
    const double f1 = fast_exp2((s.p - q2) - om), f2 = fast_exp2(kj - q2);
    s.ad = (s.ad + s.a) * f1;  // A'_{t+1} = eps (A'_t + A_t)
    s.bd = (s.bd + s.b) * f1;
    s.a = fma(s.a, f1, vj * f2);
    s.b = fma(s.b, f1, f2);
    s.p = q2;
}

// One forward step from the sums over i < t: the step's values that the reverse needs
//   c = g_t / dm (D_t = dm 2^q),  q,  y_t,  v_t - y_t,
// the step's dL/dw, dL/du terms added to sw, su, and the sums advanced past the step.
struct StepOut { float c, q, y, vmy; };

__device__ __forceinline__ StepOut fwd_step(float om, float mu, Fwd& s, float kj, float vjf, float gj,
                                            double& sw, double& su) {
    const double vj = vjf;
    const float M = mag(s.p, (float)s.b);
    const float q = ceilf(fmaxf(M, kj + mu));
    const float e1 = fast_exp2(s.p - q), e2 = fast_exp2((kj - q) + mu);
    const double dm = fma(s.b, (double)e1, (double)e2);
    const float inv = __builtin_amdgcn_rcpf((float)dm);
    const float y = (float)fma(s.a, (double)e1, vj * e2) * inv;
    const float vmy = e1 * (float)fma(vj, s.b, -s.a) * inv;
    const float c = gj * inv;
    sw -= (double)(c * e1) * fma(-(double)y, s.bd, s.ad);
    su += (double)(c * e2 * vmy);
    fwd_advance(om, s, kj, vj, M);
    return {c, q, y, vmy};
}

// Reverse sums (G, H) of a chunk of n steps seen from its first step: weights
// 2^{-q_j - j om} on c_j (and c_j y_j).
template <int L, int VEC>
__device__ __forceinline__ Rev rev_chunk(float om, const float (&qs)[L][VEC], const float (&cg)[L][VEC],
                                         const float (&ys)[L][VEC], int e, int n) {
    Rev s = rev_identity();
    if (n <= 0) return s;
    float m[L];
    float mx = kEmpty;
#pragma unroll
    for (int j = 0; j < L; ++j) {
        m[j] = (j < n) ? fmaf(-(float)j, om, -qs[j][e]) : kEmpty;
        mx = fmaxf(mx, m[j]);
    }
    s.r = ceilf(mx);
#pragma unroll
    for (int j = 0; j < L; ++j) {
        const float wgt = fast_exp2(m[j] - s.r);  // 0 for the unused slots
        const double f = wgt * cg[j][e];
        s.x += f;
        s.h = fma(f, (double)ys[j][e], s.h);
        s.z += wgt;
    }
    return s;
}

// One reverse step at time t: s holds the reverse sums over the steps after t.  Writes
// dL/dk_t, dL/dv_t, then extends s by step t.
__device__ __forceinline__ void rev_step(float om, float mu, Rev& s, float kj, float vj, float c, float q,
                                         float y, float vmy, float& gk, float& gv) {
    const float sc = fast_exp2(s.r + kj);            // alpha_t at the state's scale
    const float dgv = c * fast_exp2((kj - q) + mu);  // g_t beta_t / D_t
    gv = (float)fma(s.x, (double)sc, (double)dgv);
    gk = fmaf(dgv, vmy, sc * (float)fma((double)vj, s.x, -s.h));
    const float r2 = ceilf(fmaxf(mag(s.r, (float)s.z) - om, -q));
    const double f1 = fast_exp2((s.r - r2) - om);
    const float w2 = fast_exp2(-q - r2);
    const double f2 = w2 * c;
    s.x = fma(s.x, f1, f2);
    s.h = fma(s.h, f1, f2 * y);
    s.z = fma(s.z, f1, (double)w2);
    s.r = r2;
}

template <int VEC>
__device__ __forceinline__ void load_chan(const WkvBwdArgs& A, int64_t c0, bool active, float (&om)[VEC],
                                          float (&mu)[VEC]) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        om[e] = active ? fminf(A.w[c0 + e] * kLog2e, kMaxOm) : 0.f;
        mu[e] = active ? A.u[c0 + e] * kLog2e : 0.f;
    }
}

// The forward-state chain of sequence gi (channel group of one batch row).
template <int VEC>
__device__ __forceinline__ Chain<Fwd> fwd_chain(const BwdGeom& g, int64_t gi) {
    constexpr int64_t per = 64 * VEC * kDwords<Fwd>;  // dwords per slab record
    return {g.flags_f + gi * g.nslab, reinterpret_cast<uint32_t*>(g.agg_f) + gi * g.nslab * per,
            reinterpret_cast<uint32_t*>(g.incl_f) + gi * g.nslab * per, g.tag_f, g.spin};
}

// Forward sums at the start of slab s: the state kernel's inclusive prefix of slab s-1.
template <int VEC>
__device__ __forceinline__ void fwd_carry_in(const BwdGeom& g, int64_t gi, int64_t s, int lane, bool active,
                                             Fwd (&x)[VEC]) {
    if (s > 0 && active) {
        load_record<VEC>(fwd_chain<VEC>(g, gi).incl, s - 1, lane, x);
    } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[e] = fwd_identity();
    }
}

// Steps of chunk x of a slab of slab_n steps (0 for chunks past the end).
template <int L>
__device__ __forceinline__ int chunk_len(int x, int slab_n) {
    return max(0, min(L, slab_n - x * L));
}

// ------------------------------------------------------------------------------------
// State kernel: forward sums at the end of slabs 0 .. nslab-2.  Waves 0 .. NW-1 reduce one
// chunk each; wave NW (the coordinator) folds the chunks in order, publishes the slab's
// aggregate, looks back over the earlier slabs and publishes the inclusive prefix.
// ------------------------------------------------------------------------------------
template <int VEC, int NW, int L>
__global__ __launch_bounds__(64 * (NW + 1)) void wkv_bwd_state_kernel(WkvBwdArgs A, BwdGeom g) {
    constexpr int CW = 64 * VEC;
    constexpr int SLAB = NW * L;
    __shared__ Fwd shf[NW][CW];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int64_t G = g.B * g.ngrp;
    const int64_t s = (int64_t)blockIdx.x / G;  // slab (time order), s < nslab - 1: always full
    const int64_t gi = (int64_t)blockIdx.x - s * G;
    const int64_t b = gi / g.ngrp, grp = gi - b * g.ngrp;
    const int64_t c0 = grp * CW + (int64_t)lane * VEC;
    const bool active = c0 < g.C;  // C is a multiple of VEC

    float om[VEC], mu[VEC];
    load_chan<VEC>(A, c0, active, om, mu);

    const unsigned rowb = (unsigned)(g.C * 4);
    const unsigned voff = (unsigned)(lane * VEC * 4);
    const int64_t total = g.B * g.T * g.C;
    if (w < NW) {
        const int n = active ? L : 0;
        const int64_t base = (b * g.T + s * SLAB + (int64_t)w * L) * g.C + grp * CW;
        const rsrc_t rk = make_rsrc(A.k + base, (total - base) * 4), rv = make_rsrc(A.v + base, (total - base) * 4);
        float kk[L][VEC], vv[L][VEC];
#pragma unroll
        for (int j = 0; j < L; ++j) {
            FV<VEC> kt{}, vt{};
            if (n > 0) {
                kt = ldb<VEC>(rk, voff, j * rowb);
                vt = ldb<VEC>(rv, voff, j * rowb);
            }
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                kk[j][e] = kt.v[e] * kLog2e;
                vv[j][e] = vt.v[e];
            }
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) shf[w][lane * VEC + e] = fwd_chunk<L, VEC>(om[e], kk, vv, e, n);
        __syncthreads();
        return;
    }

    // Coordinator.
    __syncthreads();
    Fwd mine[VEC], carry[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        mine[e] = shf[0][lane * VEC + e];
        for (int x = 1; x < NW; ++x) mine[e] = fwd_combine(om[e], mine[e], shf[x][lane * VEC + e], L);
        carry[e] = fwd_identity();
    }
    const Chain<Fwd> chn = fwd_chain<VEC>(g, gi);
    publish<VEC>(chn, s, lane, mine, false);
    auto fold = [&](Fwd (&c)[VEC], const Fwd (&x)[VEC], int64_t) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) c[e] = fwd_combine(om[e], c[e], x[e], SLAB);
    };
    auto recompute = [&](int64_t jj, Fwd (&x)[VEC]) {
        const int64_t bj = (b * g.T + jj * SLAB) * g.C + grp * CW;
        const rsrc_t rkj = make_rsrc(A.k + bj, (total - bj) * 4), rvj = make_rsrc(A.v + bj, (total - bj) * 4);
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[e] = fwd_identity();
        if (active) {
            for (int t = 0; t < SLAB; ++t) {
                const FV<VEC> kt = ldb<VEC>(rkj, voff, t * rowb), vt = ldb<VEC>(rvj, voff, t * rowb);
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float kj = kt.v[e] * kLog2e;
                    fwd_advance(om[e], x[e], kj, (double)vt.v[e], mag(x[e].p, (float)x[e].b));
                }
            }
        }
    };
    look_back<VEC, 2>(chn, s, lane, carry, fold, recompute);
    Fwd incl[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) incl[e] = fwd_combine(om[e], carry[e], mine[e], SLAB);
    publish<VEC>(chn, s, lane, incl, true);
}

// The reverse record of chain slab jj computed from its inputs (the look-back's fallback
// when the slab has not published in time): the slab's forward re-run from the state
// kernel's sums, one step at a time, accumulating its reverse sums in time order.
template <int VEC, int SLAB>
__device__ __forceinline__ void rev_record_from_inputs(const WkvBwdArgs& A, const BwdGeom& g, int64_t jj,
                                                       int64_t gi, int64_t b, int64_t grp, int lane, bool active,
                                                       const float (&om)[VEC], const float (&mu)[VEC],
                                                       RevRec (&x)[VEC]) {
    constexpr int CW = 64 * VEC;
    const int64_t sj = g.nslab - 1 - jj;
    const int nj = (int)((g.T - sj * SLAB) < SLAB ? (g.T - sj * SLAB) : SLAB);
    const int64_t total = g.B * g.T * g.C;
    const int64_t bj = (b * g.T + sj * SLAB) * g.C + grp * CW;
    const unsigned rowb = (unsigned)(g.C * 4);
    const unsigned voff = (unsigned)(lane * VEC * 4);
    const rsrc_t rkj = make_rsrc(A.k + bj, (total - bj) * 4), rvj = make_rsrc(A.v + bj, (total - bj) * 4),
                 rgj = make_rsrc(A.gy + bj, (total - bj) * 4);
    Fwd fs[VEC];
    fwd_carry_in<VEC>(g, gi, sj, lane, active, fs);
#pragma unroll
    for (int e = 0; e < VEC; ++e) x[e] = {rev_identity(), 0.0, 0.0};
    if (!active) return;
    for (int t = 0; t < nj; ++t) {
        const FV<VEC> kt = ldb<VEC>(rkj, voff, t * rowb), vt = ldb<VEC>(rvj, voff, t * rowb),
                      gt = ldb<VEC>(rgj, voff, t * rowb);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const StepOut o = fwd_step(om[e], mu[e], fs[e], kt.v[e] * kLog2e, vt.v[e], gt.v[e], x[e].sw, x[e].su);
            const Rev one{(double)o.c, (double)o.c * (double)o.y, 1.0, -o.q};
            x[e].st = rev_combine(om[e], one, x[e].st, t);
        }
    }
}

// ------------------------------------------------------------------------------------
// Gradient kernel: slabs in reverse time order (chain position q = nslab-1-s).  Waves
// 0 .. NW-1 own one chunk each and hold its inputs and per-step values in registers; wave
// NW (the coordinator) turns the chunk sums into carries between the compute phases:
//   B1  chunks' forward sums in shf      -> coordinator: carry-in of each chunk, in shf
//   B3  chunks' reverse sums in shr, and -> coordinator: slab record, look-back over the
//       their dL/dw, dL/du in shwu           later slabs, reverse state at each chunk end, in shr
// The two roles are separate branches, so the look-back's registers do not add to those
// of the chunk data.
// ------------------------------------------------------------------------------------
template <int VEC, int NW, int L>
__global__ __launch_bounds__(64 * (NW + 1)) void wkv_bwd_grad_kernel(WkvBwdArgs A, BwdGeom g) {
    constexpr int CW = 64 * VEC;
    constexpr int SLAB = NW * L;
    __shared__ Fwd shf[NW][CW];
    __shared__ Rev shr[NW][CW];
    __shared__ double shwu[NW][CW][2];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int64_t G = g.B * g.ngrp;
    const int64_t q = (int64_t)blockIdx.x / G;  // chain position: later slabs first
    const int64_t gi = (int64_t)blockIdx.x - q * G;
    const int64_t s = g.nslab - 1 - q;
    const int64_t b = gi / g.ngrp, grp = gi - b * g.ngrp;
    const int64_t c0 = grp * CW + (int64_t)lane * VEC;
    const bool active = c0 < g.C;
    const int64_t t_slab = s * SLAB;
    const int slab_n = (int)((g.T - t_slab) < SLAB ? (g.T - t_slab) : SLAB);

    float om[VEC], mu[VEC];
    load_chan<VEC>(A, c0, active, om, mu);

    if (w < NW) {
        const int n = active ? chunk_len<L>(w, slab_n) : 0;
        const unsigned rowb = (unsigned)(g.C * 4);
        const unsigned voff = (unsigned)(lane * VEC * 4);
        const int64_t total = g.B * g.T * g.C;
        const int64_t base = (b * g.T + t_slab + (int64_t)w * L) * g.C + grp * CW;
        const int64_t nbytes = (total - base) * 4;
        float kk[L][VEC], vv[L][VEC], gg[L][VEC];
        {
            const rsrc_t rk = make_rsrc(A.k + base, nbytes), rv = make_rsrc(A.v + base, nbytes),
                         rg = make_rsrc(A.gy + base, nbytes);
#pragma unroll
            for (int j = 0; j < L; ++j) {
                FV<VEC> kt{}, vt{}, gt{};
                if (j < n) {
                    kt = ldb<VEC>(rk, voff, j * rowb);
                    vt = ldb<VEC>(rv, voff, j * rowb);
                    gt = ldb<VEC>(rg, voff, j * rowb);
                }
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    kk[j][e] = kt.v[e] * kLog2e;
                    vv[j][e] = vt.v[e];
                    gg[j][e] = gt.v[e];
                }
            }
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) shf[w][lane * VEC + e] = fwd_chunk<L, VEC>(om[e], kk, vv, e, n);
        __syncthreads();  // B1
        __syncthreads();  // B2: shf[w] now holds my chunk's carry-in

        // Forward re-run: per step c, q, y, v - y (the registers of g are reused for c).
        float qs[L][VEC], ys[L][VEC], dv[L][VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            Fwd st = shf[w][lane * VEC + e];
            double sw = 0.0, su = 0.0;
#pragma unroll
            for (int j = 0; j < L; ++j) {
                if (j < n) {
                    const StepOut o = fwd_step(om[e], mu[e], st, kk[j][e], vv[j][e], gg[j][e], sw, su);
                    gg[j][e] = o.c;
                    qs[j][e] = o.q;
                    ys[j][e] = o.y;
                    dv[j][e] = o.vmy;
                } else {
                    gg[j][e] = 0.f;
                    qs[j][e] = 0.f;
                    ys[j][e] = 0.f;
                    dv[j][e] = 0.f;
                }
            }
            shwu[w][lane * VEC + e][0] = sw;
            shwu[w][lane * VEC + e][1] = su;
            shr[w][lane * VEC + e] = rev_chunk<L, VEC>(om[e], qs, gg, ys, e, n);
        }
        __syncthreads();  // B3
        __syncthreads();  // B4: shr[w] now holds the reverse state at my chunk's end

        // Reverse re-run of my chunk; the outputs replace k and v.
        if (n > 0) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                Rev rs = shr[w][lane * VEC + e];
#pragma unroll
                for (int j = L - 1; j >= 0; --j) {
                    if (j < n) {
                        float gk, gv;
                        rev_step(om[e], mu[e], rs, kk[j][e], vv[j][e], gg[j][e], qs[j][e], ys[j][e], dv[j][e], gk, gv);
                        kk[j][e] = gk;
                        vv[j][e] = gv;
                    }
                }
            }
            const rsrc_t rgk = make_rsrc(A.gk + base, nbytes), rgv = make_rsrc(A.gv + base, nbytes);
#pragma unroll
            for (int j = 0; j < L; ++j) {
                if (j < n) {
                    FV<VEC> ok, ov;
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        ok.v[e] = kk[j][e];
                        ov.v[e] = vv[j][e];
                    }
                    stb<VEC>(rgk, voff, j * rowb, ok);
                    stb<VEC>(rgv, voff, j * rowb, ov);
                }
            }
        }
        return;
    }

    // ---- coordinator ----
    __syncthreads();  // B1
    {
        // Carry-in of each chunk: the previous slab's sums (state kernel), then the chunks in order.
        Fwd cin[VEC];
        fwd_carry_in<VEC>(g, gi, s, lane, active, cin);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            Fwd c = cin[e];
            for (int x = 0; x < NW; ++x) {
                const Fwd chunk = shf[x][lane * VEC + e];
                shf[x][lane * VEC + e] = c;
                c = fwd_combine(om[e], c, chunk, chunk_len<L>(x, slab_n));
            }
        }
    }
    __syncthreads();  // B2
    __syncthreads();  // B3
    RevRec mine[VEC], carry[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        // Reverse sums of the slab from its start: chunks folded from the last to the first.
        Rev a = rev_identity();
        double sw = 0.0, su = 0.0;
        for (int x = NW - 1; x >= 0; --x) a = rev_combine(om[e], a, shr[x][lane * VEC + e], chunk_len<L>(x, slab_n));
        for (int x = 0; x < NW; ++x) {
            sw += shwu[x][lane * VEC + e][0];
            su += shwu[x][lane * VEC + e][1];
        }
        mine[e] = {a, sw, su};
        carry[e] = {rev_identity(), 0.0, 0.0};
    }
    const Chain<RevRec> chn{g.flags_r + gi * g.nslab,
                            reinterpret_cast<uint32_t*>(g.agg_r) + gi * g.nslab * (CW * kDwords<RevRec>),
                            reinterpret_cast<uint32_t*>(g.incl_r) + gi * g.nslab * (CW * kDwords<RevRec>), g.tag_r,
                            g.spin};
    const bool has_succ = s > 0;
    if (has_succ) publish<VEC>(chn, q, lane, mine, false);
    // carry (the state at the end of chain slab jj) followed by slab jj, earlier in time.
    auto fold = [&](RevRec (&cr)[VEC], const RevRec (&x)[VEC], int64_t jj) {
        const int64_t sj = g.nslab - 1 - jj;
        const int64_t len = (g.T - sj * SLAB) < SLAB ? (g.T - sj * SLAB) : SLAB;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            cr[e].st = rev_combine(om[e], cr[e].st, x[e].st, len);
            cr[e].sw += x[e].sw;
            cr[e].su += x[e].su;
        }
    };
    auto recompute = [&](int64_t jj, RevRec (&x)[VEC]) {
        rev_record_from_inputs<VEC, SLAB>(A, g, jj, gi, b, grp, lane, active, om, mu, x);
    };
    look_back<VEC, 2>(chn, q, lane, carry, fold, recompute);
    RevRec incl[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) incl[e] = carry[e];
    fold(incl, mine, q);
    if (has_succ) {
        publish<VEC>(chn, q, lane, incl, true);
    } else if (active) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            g.part[2 * (b * g.C + c0 + e)] = incl[e].sw;
            g.part[2 * (b * g.C + c0 + e) + 1] = incl[e].su;
        }
    }
    // Reverse state at the end of each chunk: from the slab's end, backwards.
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        Rev r = carry[e].st;
        for (int x = NW - 1; x >= 0; --x) {
            const Rev chunk = shr[x][lane * VEC + e];
            shr[x][lane * VEC + e] = r;
            r = rev_combine(om[e], r, chunk, chunk_len<L>(x, slab_n));
        }
    }
    __syncthreads();  // B4
}

// gw[c] = sum_b part[b, c].w, gu likewise, in ascending b.
__global__ __launch_bounds__(256) void wkv_bwd_wu_kernel(const double* __restrict__ part, int64_t B,
                                                         int64_t C, float* __restrict__ gw,
                                                         float* __restrict__ gu) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= C) return;
    double sw = 0.0, su = 0.0;
    for (int64_t b = 0; b < B; ++b) {
        sw += part[2 * (b * C + c)];
        su += part[2 * (b * C + c) + 1];
    }
    gw[c] = (float)sw;
    gu[c] = (float)su;
}

__global__ __launch_bounds__(256) void zero_wu_kernel(float* __restrict__ gw, float* __restrict__ gu,
                                                      int64_t C) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c < C) {
        gw[c] = 0.f;
        gu[c] = 0.f;
    }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <int VEC, int NW, int L>
hipError_t launch(const WkvBwdArgs& A, const BwdGeom& g, hipStream_t st) {
    const int64_t G = g.B * g.ngrp;
    if (g.nslab > 1) {
        hipLaunchKernelGGL((wkv_bwd_state_kernel<VEC, NW, L>), dim3((unsigned)(G * (g.nslab - 1))), dim3(64 * (NW + 1)),
                           0, st, A, g);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((wkv_bwd_grad_kernel<VEC, NW, L>), dim3((unsigned)(G * g.nslab)), dim3(64 * (NW + 1)), 0, st,
                       A, g);
    return hipGetLastError();
}

// Kernels that exist (one channel per lane): (nw, L) in {(3, 16), (4, 16), (7, 8), (8, 8), (7, 16)}.
hipError_t dispatch_shape(const WkvBwdArgs& A, const BwdGeom& g, const BwdPlan& p, hipStream_t st) {
    if (p.nw == 3 && p.L == 16) return launch<1, 3, 16>(A, g, st);
    if (p.nw == 4 && p.L == 16) return launch<1, 4, 16>(A, g, st);
    if (p.nw == 7 && p.L == 8) return launch<1, 7, 8>(A, g, st);
    if (p.nw == 8 && p.L == 8) return launch<1, 8, 8>(A, g, st);
    if (p.nw == 7 && p.L == 16) return launch<1, 7, 16>(A, g, st);
    return hipErrorInvalidValue;
}

}  // namespace

bool bwd_shape_supported(int vec, int nw, int L) {
    return vec == 1 && ((nw == 3 && L == 16) || (nw == 4 && L == 16) || (nw == 7 && L == 8) || (nw == 8 && L == 8) ||
                        (nw == 7 && L == 16));
}

BwdPlan wkv_backward_plan(int vec, int64_t B, int64_t T, int64_t C, int nw_override, int L_override) {
    BwdPlan p{};
    // One channel per lane (256-byte rows): the gradient kernel keeps six float32 values per
    // step in registers, and two channels per lane would not fit.  7 compute waves plus the
    // coordinator make 8-wave workgroups, two of which fit on a CU at <= 128 VGPRs.
    p.vec = vec = 1;
    p.nw = 7;
    p.L = 8;
    if (nw_override > 0 && L_override > 0 && bwd_shape_supported(vec, nw_override, L_override)) {
        p.nw = nw_override;
        p.L = L_override;
    }
    const int64_t slab = (int64_t)p.nw * p.L;
    p.nslab = (T + slab - 1) / slab;
    const int64_t cw = 64 * (int64_t)vec;
    const int64_t nrec = B * ((C + cw - 1) / cw) * p.nslab;
    size_t bytes = align256((size_t)(B * C) * 2 * sizeof(double));  // part
    if (p.nslab > 1) {
        bytes += 2 * align256((size_t)nrec * 8);                           // flags
        bytes += 2 * align256((size_t)(nrec * cw) * sizeof(Fwd));          // forward records
        bytes += 2 * align256((size_t)(nrec * cw) * sizeof(RevRec));       // reverse records
    }
    p.ws_bytes = bytes;
    return p;
}

void wkv_backward_layout(const BwdPlan& p, int64_t B, int64_t C, void* ws, BwdGeom& g) {
    char* at = (char*)ws;
    g.part = reinterpret_cast<double*>(at);
    at += align256((size_t)(B * C) * 2 * sizeof(double));
    g.flags_f = g.flags_r = nullptr;
    g.agg_f = g.incl_f = g.agg_r = g.incl_r = nullptr;
    if (p.nslab <= 1) return;
    const int64_t cw = 64 * (int64_t)p.vec;
    const int64_t nrec = B * ((C + cw - 1) / cw) * p.nslab;
    const size_t fl = align256((size_t)nrec * 8);
    const size_t fr = align256((size_t)(nrec * cw) * sizeof(Fwd));
    const size_t rr = align256((size_t)(nrec * cw) * sizeof(RevRec));
    g.flags_f = reinterpret_cast<uint64_t*>(at), at += fl;
    g.flags_r = reinterpret_cast<uint64_t*>(at), at += fl;
    g.agg_f = at, at += fr;
    g.incl_f = at, at += fr;
    g.agg_r = at, at += rr;
    g.incl_r = at;
}

hipError_t run_wkv_backward(const WkvBwdArgs& A, const BwdGeom& g, const BwdPlan& p, hipStream_t st) {
    const hipError_t e = dispatch_shape(A, g, p, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(wkv_bwd_wu_kernel, dim3((unsigned)((g.C + 255) / 256)), dim3(256), 0, st, g.part, g.B, g.C,
                       A.gw, A.gu);
    return hipGetLastError();
}

hipError_t run_zero_wu(float* gw, float* gu, int64_t C, hipStream_t st) {
    hipLaunchKernelGGL(zero_wu_kernel, dim3((unsigned)((C + 255) / 256)), dim3(256), 0, st, gw, gu, C);
    return hipGetLastError();
}

}  // namespace linrec

// scan_ops.hpp -- the three first-order recurrences as operators of the chunked scan.
//
// Each operator supplies, for one channel:
//   Chan     per-channel constants,
//   In       one time step's inputs (loaded with channel-contiguous vector loads),
//   Agg      the state after a span of steps, and the span's effect on an incoming state,
//   reduce   the aggregate of a chunk of n <= L steps started from the identity,
//   combine  aggregate(s1 then s2) given the n2 steps s2 covers (s1 is earlier in the
//            recurrence's order),
//   run      the chunk's steps from an incoming state, writing one output per step, and
//            returning the lane's share of any per-slab sum (Part; empty for most).
// Steps are addressed through Rows (chunk_scan.hpp): kReverse operators run backwards in
// time, so their logical step j is time t0 - j.
// Each combine is associative, which is what lets a sequence be cut into chunks whose
// aggregates are scanned and then re-run from their carries (the two-halves split of the
// LRU write-up, parallelisation section: x_T = lam^{T-t} x_t + local sum over (t, T]).
#pragma once

#include <type_traits>

#include "chunk_scan.hpp"
#include "device_common.hpp"
#include "wkv_math.hpp"

namespace linrec {

// ----------------------------------------------------------------------------------
// WKV-4, RWKV-LLM page "Time-mixing block", eq. (14).
// The past sums A_t = sum_{i<t} e^{-(t-1-i)w + k_i} v_i and B_t (same without v) are kept
// as (a, b, p): A = a 2^p, B = b 2^p, p an integer exponent (see wkv_math.hpp), in base 2
// (kk = k log2 e, om = w log2 e, mu = u log2 e).
//
// Phase 1 (chunk of n steps from the empty state): m_j = kk_j - (n-1-j) om is the exponent
// of step j's weight at the chunk end; p = ceil(max_j m_j), g_j = 2^{m_j - p} <= 1, and the
// aggregate is (sum g_j v_j, sum g_j, p).  The g_j stay in registers (replacing kk_j).
//
// Phase 3 re-runs the chunk from its carry (a0, b0, p0).  Fast path: a frame that decays
// with the sums, A~_j = A_{t0+j} 2^{-F_0 + j om}, turns the recurrence into plain sums,
//   A~_{j+1} = A~_j + 2^{om-D} g_j v_j,   y_j = (A~_j + 2^{mu-D} g_j v_j) / (B~_j + 2^{mu-D} g_j),
// with F_0 = p + (n-1) om + D and D >= max(om, mu, 0) chosen so no term exceeds 1: one
// exponential per element, shared with phase 1.  It is taken when the largest term of the
// first step's denominator is at least 2^-120 (so nothing that matters can underflow);
// otherwise the chunk runs the exact per-step running maximum with integer exponents,
//   output  q = ceil(max(M, kk_t + mu)),  y = (a 2^{p-q} + v 2^{kk+mu-q}) / (b 2^{p-q} + 2^{kk+mu-q})
//   update  p' = ceil(max(M - om, kk_t)), a <- a 2^{p-p'-om} + v 2^{kk-p'}, b likewise,
// where M = p + frexp_exp(b) bounds log2 B (see wkv_math.hpp),
// re-reading k from memory (its registers now hold g).
// ----------------------------------------------------------------------------------
// kExt: the instance that reads a carried state, writes the final one and gates the output by
// sigma(r).  The plain instance compiles none of that, so its registers stay as they were.
struct NoPart {};

template <bool kExt>
struct WkvOpT {
    using Args = WkvArgs;
    static constexpr bool kReverse = false;
    static constexpr bool kParts = false;
    // Uses its lane offset only for buffer accesses: the kernel may run every lane of a wave
    // over the same step count and drop an inactive lane's accesses by an out-of-range offset
    // (see scan_kernel.hpp).
    static constexpr bool kUniformSteps = true;
    static constexpr bool kChanLate = true;  // w, u are read after the chunk's loads are issued
    using Part = NoPart;
    struct Chan { float om, mu, lift, fast_lo; };  // lift = ceil(max(om, mu, 0))
    // kk becomes g_j after phase 1.  The gated instance also loads r with the chunk, so that
    // its loads are in flight with k and v instead of after the look-back.
    struct InPlain { float kk, v; };
    struct InGated { float kk, v, r; };
    using In = typename std::conditional<kExt, InGated, InPlain>::type;
    struct Local { float p, m0; };        // chunk exponent p and m_0 - p
    struct Agg { float a, b, p; };

    template <int L>
    __device__ __forceinline__ static Chan chan(const Args& A, int64_t c) {
        Chan ch;
        ch.om = fminf(A.w[c] * kLog2e, kMaxOm);
        ch.mu = A.u[c] * kLog2e;
        ch.lift = ceilf(fmaxf(fmaxf(ch.om, ch.mu), 0.f));
        ch.fast_lo = A.exact_only ? __builtin_inff() : -120.f;
        return ch;
    }
    __device__ __forceinline__ static Agg identity() { return {0.f, 0.f, kEmpty}; }

    // A carried state (a, b, p) in natural log (see wkv_math.hpp), read before the first
    // token and written after the last.
    __device__ __forceinline__ static Agg init(const Args& A, const ScanGeom& g, int64_t b, int64_t c) {
        if constexpr (!kExt) {
            return identity();
        } else {
            if (!A.s_in) return identity();
            const float* s = A.s_in + 3 * (b * g.C + c);
            const Base2State x = state_from_natural(s[0], s[1], s[2]);
            return {x.a, x.b, x.p};
        }
    }
    __device__ __forceinline__ static void finish(const Args& A, const ScanGeom& g, int64_t b, int64_t c,
                                                  const Agg& s) {
        if constexpr (kExt) {
            if (!A.s_out) return;
            float* o = A.s_out + 3 * (b * g.C + c);
            state_to_natural({s.a, s.b, s.p}, o[0], o[1], o[2]);
        }
    }

    static constexpr int kFloats = 1;  // floats per channel element
    struct Res { rsrc_t k, v, y, r; bool gated; };
    // Buffers of the run whose lowest row is time `row` of batch row b, from column col0.
    __device__ __forceinline__ static Res res(const Args& A, const ScanGeom& g, int64_t b, int64_t row, int64_t col0) {
        const int64_t base = (b * g.T + row) * g.C + col0, nbytes = (g.B * g.T * g.C - base) * 4;
        return {make_rsrc(A.k + base, nbytes), make_rsrc(A.v + base, nbytes), make_rsrc(A.y + base, nbytes),
                make_rsrc(A.r ? A.r + base : A.k + base, A.r ? nbytes : 0), A.r != nullptr};
    }
    // sigma(r) of the gated output (eq. (15)); 1 without a gate.
    template <int L, int VEC>
    __device__ __forceinline__ static void gates(const Res& R, const In (&in)[L][VEC], float (&sg)[L][VEC]) {
#pragma unroll
        for (int j = 0; j < L; ++j)
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                if constexpr (kExt) {
                    sg[j][e] = R.gated ? __builtin_amdgcn_rcpf(1.f + fast_exp2(-in[j][e].r * kLog2e)) : 1.f;
                } else {
                    sg[j][e] = 1.f;
                }
            }
    }
    template <int VEC>
    __device__ __forceinline__ static void load(const Res& R, unsigned voff, const Rows& rows, int j, In (&in)[VEC]) {
        const FV<VEC> k = ldb<VEC>(R.k, voff, rows.soff(j));
        const FV<VEC> v = ldb<VEC>(R.v, voff, rows.soff(j));
        if constexpr (kExt) {
            FV<VEC> r{};
            if (R.gated) r = ldb<VEC>(R.r, voff, rows.soff(j));
#pragma unroll
            for (int e = 0; e < VEC; ++e) in[e] = {k.v[e] * kLog2e, v.v[e], r.v[e]};
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) in[e] = {k.v[e] * kLog2e, v.v[e]};
        }
    }
    template <int VEC>
    __device__ __forceinline__ static void zero(In (&in)[VEC]) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) in[e] = In{};
    }

    template <int L, int VEC>
    __device__ __forceinline__ static Agg reduce(const Chan& ch, In (&in)[L][VEC], int e, int n, Local& loc) {
        if (n <= 0) {
            loc = {kEmpty, kEmpty};
            return identity();
        }
        float m[L];
        float mx = kEmpty;
#pragma unroll
        for (int j = 0; j < L; ++j) {
            m[j] = (j < n) ? fmaf(-(float)(n - 1 - j), ch.om, in[j][e].kk) : kEmpty;
            mx = fmaxf(mx, m[j]);
        }
        const float p = ceilf(mx);
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int j = 0; j < L; ++j) {
            const float g = fast_exp2(m[j] - p);  // 0 for the unused slots
            in[j][e].kk = g;
            a = fmaf(g, in[j][e].v, a);
            b += g;
        }
        loc = {p, m[0] - p};
        return {a, b, p};
    }

    __device__ __forceinline__ static Agg combine(const Chan& ch, const Agg& s1, const Agg& s2, int64_t n2) {
        float p, f1, f2;
        merge_scales(s1.p, s1.b, s2.p, s2.b, mul_split((float)n2, ch.om), p, f1, f2);
        return {fmaf(s1.a, f1, s2.a * f2), fmaf(s1.b, f1, s2.b * f2), p};
    }

    // The aggregate s extended by one step (the exact per-step update).
    __device__ __forceinline__ static Agg step(const Chan& ch, const Agg& s, const In& x) {
        const float q = ceilf(fmaxf(mag(s.p, s.b) - ch.om, x.kk));
        const float f1 = fast_exp2((s.p - q) - ch.om), f2 = fast_exp2(x.kk - q);
        return {fmaf(s.a, f1, x.v * f2), fmaf(s.b, f1, f2), q};
    }

    template <int L, int VEC>
    __device__ __forceinline__ static Part run(const Res& R, const Chan (&ch)[VEC], const Agg (&cin)[VEC],
                               const In (&in)[L][VEC], const Local (&loc)[VEC], int n, unsigned voff,
                               const Rows& rows) {
        float sg[L][VEC];
        gates<L, VEC>(R, in, sg);
        float a[VEC], b[VEC], cs[VEC], us[VEC];
        bool fast[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            // Carry exponent relative to the chunk frame: p0 - p - (n-1) om.
            const Split d = mul_split((float)(n - 1), ch[e].om);
            const float rel = ((cin[e].p - loc[e].p) - d.hi) - d.lo;
            const float fe = (float)__builtin_amdgcn_frexp_expf(cin[e].b);  // b0 < 2^fe
            const float D = fmaxf(ch[e].lift, rel + fe);
            const float carry_lo = (rel + fe - 1.f) - D;       // log2 of the carry's size, >=
            const float cur_lo = (loc[e].m0 + ch[e].mu) - D;   // log2 of step 0's own weight
            fast[e] = fmaxf(carry_lo, cur_lo) >= ch[e].fast_lo;
            const float cf = fast_exp2(rel - D);
            a[e] = cin[e].a * cf;
            b[e] = cin[e].b * cf;
            cs[e] = fast_exp2(ch[e].mu - D);
            us[e] = fast_exp2(ch[e].om - D);
        }
        bool all_fast = true;
#pragma unroll
        for (int e = 0; e < VEC; ++e) all_fast = all_fast && fast[e];
        if (all_fast) {
#pragma unroll
            for (int j = 0; j < L; ++j) {
                if (j < n) {
                    FV<VEC> y;
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        const float g = in[j][e].kk, vv = in[j][e].v;
                        const float cur = g * cs[e];
                        y.v[e] = fmaf(cur, vv, a[e]) * __builtin_amdgcn_rcpf(b[e] + cur) * sg[j][e];
                        const float up = g * us[e];
                        a[e] = fmaf(up, vv, a[e]);
                        b[e] += up;
                    }
                    stb<VEC>(R.y, voff, rows.soff(j), y);
                }
            }
            return {};
        }
        // Exact per-step running maximum (integer exponents), all channels of the lane.
        float pa[VEC], pb[VEC], pp[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) { pa[e] = cin[e].a; pb[e] = cin[e].b; pp[e] = cin[e].p; }
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                const FV<VEC> kr = ldb<VEC>(R.k, voff, rows.soff(j));
                FV<VEC> y;
    #pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float kk = kr.v[e] * kLog2e, vv = in[j][e].v;
                    const float q = ceilf(fmaxf(mag(pp[e], pb[e]), kk + ch[e].mu));
                    const float e1 = fast_exp2(pp[e] - q), e2 = fast_exp2((kk - q) + ch[e].mu);
                    y.v[e] = fmaf(pa[e], e1, vv * e2) * __builtin_amdgcn_rcpf(fmaf(pb[e], e1, e2)) * sg[j][e];
                    const float q2 = ceilf(fmaxf(mag(pp[e], pb[e]) - ch[e].om, kk));
                    const float f1 = fast_exp2((pp[e] - q2) - ch[e].om), f2 = fast_exp2(kk - q2);
                    pa[e] = fmaf(pa[e], f1, vv * f2);
                    pb[e] = fmaf(pb[e], f1, f2);
                    pp[e] = q2;
                }
                stb<VEC>(R.y, voff, rows.soff(j), y);
            }
        }
        return {};
    }
};
using WkvOp = WkvOpT<false>;
using WkvExtOp = WkvOpT<true>;

// ----------------------------------------------------------------------------------
// Real diagonal scan x_t = a_t x_{t-1} + b_t ("Were RNNs All We Needed?" page, minGRU
// section).  Aggregate of a span: (m, x) = (product of its a, its output from x = 0);
// (m1, x1) then (m2, x2) is (m1 m2, m2 x1 + x2).
// ----------------------------------------------------------------------------------


struct RealOp {
    using Args = RealArgs;
    static constexpr bool kReverse = false;
    static constexpr bool kParts = false;
    using Part = NoPart;
    // The final state is the last row of x: nothing more to write.
    template <class AnyArgs, class AnyAgg>
    __device__ __forceinline__ static void finish(const AnyArgs&, const ScanGeom&, int64_t, int64_t, const AnyAgg&) {}
    struct Chan {};
    struct In { float a, b; };
    struct Local {};
    struct Agg { float m, x; };

    template <int L>
    __device__ __forceinline__ static Chan chan(const Args&, int64_t) { return {}; }
    __device__ __forceinline__ static Agg identity() { return {1.f, 0.f}; }
    __device__ __forceinline__ static Agg init(const Args& A, const ScanGeom& g, int64_t b, int64_t c) {
        return {1.f, A.x0 ? A.x0[b * g.C + c] : 0.f};
    }

    static constexpr int kFloats = 1;
    struct Res { rsrc_t a, b, x; };
    __device__ __forceinline__ static Res res(const Args& A, const ScanGeom& g, int64_t b, int64_t row, int64_t col0) {
        const int64_t base = (b * g.T + row) * g.C + col0, nbytes = (g.B * g.T * g.C - base) * 4;
        return {make_rsrc(A.a + base, nbytes), make_rsrc(A.b + base, nbytes), make_rsrc(A.x + base, nbytes)};
    }
    template <int VEC>
    __device__ __forceinline__ static void load(const Res& R, unsigned voff, const Rows& rows, int j, In (&in)[VEC]) {
        const FV<VEC> a = ldb<VEC>(R.a, voff, rows.soff(j));
        const FV<VEC> b = ldb<VEC>(R.b, voff, rows.soff(j));
#pragma unroll
        for (int e = 0; e < VEC; ++e) in[e] = {a.v[e], b.v[e]};
    }
    template <int VEC>
    __device__ __forceinline__ static void zero(In (&in)[VEC]) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) in[e] = {1.f, 0.f};
    }

    template <int L, int VEC>
    __device__ __forceinline__ static Agg reduce(const Chan&, In (&in)[L][VEC], int e, int n, Local&) {
        float m = 1.f, x = 0.f;
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                x = fmaf(in[j][e].a, x, in[j][e].b);
                m *= in[j][e].a;
            }
        }
        return {m, x};
    }

    __device__ __forceinline__ static Agg combine(const Chan&, const Agg& s1, const Agg& s2, int64_t) {
        return {s1.m * s2.m, fmaf(s2.m, s1.x, s2.x)};
    }

    __device__ __forceinline__ static Agg step(const Chan&, const Agg& s, const In& x) {
        return {s.m * x.a, fmaf(x.a, s.x, x.b)};
    }

    // RS: any buffer set with the output x (the gated variants below bring their own).
    template <int L, int VEC, class RS>
    __device__ __forceinline__ static Part run(const RS& R, const Chan (&)[VEC], const Agg (&cin)[VEC],
                               const In (&in)[L][VEC], const Local (&)[VEC], int n, unsigned voff,
                               const Rows& rows) {
        float x[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[e] = cin[e].x;
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                FV<VEC> o;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    x[e] = fmaf(in[j][e].a, x[e], in[j][e].b);
                    o.v[e] = x[e];
                }
                stb<VEC>(R.x, voff, rows.soff(j), o);
            }
        }
        return {};
    }
};

// ----------------------------------------------------------------------------------
// Complex diagonal scan x_t = lam x_{t-1} + u_t (LRU write-up, eq. lr-xx), complex64.
// Aggregate of a span of n steps: (lam^n, its output from x = 0).  lam^n for a full
// chunk is formed in float64 by repeated squaring from the complex64 lam.
// ----------------------------------------------------------------------------------


__device__ __forceinline__ void cpow64(double br, double bi, int64_t n, float& rr, float& ri) {
    double pr = 1.0, pi = 0.0;
    while (n > 0) {
        if (n & 1) {
            const double t = pr * br - pi * bi;
            pi = pr * bi + pi * br;
            pr = t;
        }
        const double t = br * br - bi * bi;
        bi = 2.0 * br * bi;
        br = t;
        n >>= 1;
    }
    rr = (float)pr;
    ri = (float)pi;
}

struct CplxOp {
    using Args = CplxArgs;
    static constexpr bool kReverse = false;
    static constexpr bool kParts = false;
    using Part = NoPart;
    template <class AnyArgs, class AnyAgg>
    __device__ __forceinline__ static void finish(const AnyArgs&, const ScanGeom&, int64_t, int64_t, const AnyAgg&) {}
    struct Chan { float lr, li, Lr, Li; };  // lam and lam^L
    struct In { float r, i; };
    struct Local {};
    struct Agg { float mr, mi, xr, xi; };

    template <int L>
    __device__ __forceinline__ static Chan chan(const Args& A, int64_t c) {
        Chan ch;
        ch.lr = A.lam[2 * c];
        ch.li = A.lam[2 * c + 1];
        cpow64((double)ch.lr, (double)ch.li, L, ch.Lr, ch.Li);
        return ch;
    }
    __device__ __forceinline__ static Agg identity() { return {1.f, 0.f, 0.f, 0.f}; }
    __device__ __forceinline__ static Agg init(const Args& A, const ScanGeom& g, int64_t b, int64_t c) {
        if (!A.x0) return identity();
        return {1.f, 0.f, A.x0[2 * (b * g.C + c)], A.x0[2 * (b * g.C + c) + 1]};
    }

    static constexpr int kFloats = 2;
    struct Res { rsrc_t u, x; };
    __device__ __forceinline__ static Res res(const Args& A, const ScanGeom& g, int64_t b, int64_t row, int64_t col0) {
        const int64_t base = (b * g.T + row) * g.C + col0, nbytes = (g.B * g.T * g.C - base) * 8;
        return {make_rsrc(A.u + 2 * base, nbytes), make_rsrc(A.x + 2 * base, nbytes)};
    }
    template <int VEC>
    __device__ __forceinline__ static void load(const Res& R, unsigned voff, const Rows& rows, int j, In (&in)[VEC]) {
        const FV<2 * VEC> t = ldb<2 * VEC>(R.u, voff, rows.soff(j));
#pragma unroll
        for (int e = 0; e < VEC; ++e) in[e] = {t.v[2 * e], t.v[2 * e + 1]};
    }
    template <int VEC>
    __device__ __forceinline__ static void zero(In (&in)[VEC]) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) in[e] = {0.f, 0.f};
    }

    template <int L, int VEC>
    __device__ __forceinline__ static Agg reduce(const Chan& ch, In (&in)[L][VEC], int e, int n, Local&) {
        float xr = 0.f, xi = 0.f;
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                const float tr = fmaf(ch.lr, xr, fmaf(-ch.li, xi, in[j][e].r));
                xi = fmaf(ch.lr, xi, fmaf(ch.li, xr, in[j][e].i));
                xr = tr;
            }
        }
        Agg r;
        r.xr = xr;
        r.xi = xi;
        if (n == L) {
            r.mr = ch.Lr;
            r.mi = ch.Li;
        } else {
            cpow64((double)ch.lr, (double)ch.li, n, r.mr, r.mi);
        }
        return r;
    }

    __device__ __forceinline__ static Agg step(const Chan& ch, const Agg& s, const In& x) {
        Agg r;
        r.mr = fmaf(s.mr, ch.lr, -s.mi * ch.li);
        r.mi = fmaf(s.mr, ch.li, s.mi * ch.lr);
        r.xr = fmaf(ch.lr, s.xr, fmaf(-ch.li, s.xi, x.r));
        r.xi = fmaf(ch.lr, s.xi, fmaf(ch.li, s.xr, x.i));
        return r;
    }

    __device__ __forceinline__ static Agg combine(const Chan&, const Agg& s1, const Agg& s2, int64_t) {
        Agg r;
        r.mr = fmaf(s1.mr, s2.mr, -s1.mi * s2.mi);
        r.mi = fmaf(s1.mr, s2.mi, s1.mi * s2.mr);
        r.xr = fmaf(s2.mr, s1.xr, fmaf(-s2.mi, s1.xi, s2.xr));
        r.xi = fmaf(s2.mr, s1.xi, fmaf(s2.mi, s1.xr, s2.xi));
        return r;
    }

    template <int L, int VEC>
    __device__ __forceinline__ static Part run(const Res& R, const Chan (&ch)[VEC], const Agg (&cin)[VEC],
                               const In (&in)[L][VEC], const Local (&)[VEC], int n, unsigned voff,
                               const Rows& rows) {
        float xr[VEC], xi[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) { xr[e] = cin[e].xr; xi[e] = cin[e].xi; }
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                FV<2 * VEC> o;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float tr = fmaf(ch[e].lr, xr[e], fmaf(-ch[e].li, xi[e], in[j][e].r));
                    xi[e] = fmaf(ch[e].lr, xi[e], fmaf(ch[e].li, xr[e], in[j][e].i));
                    xr[e] = tr;
                    o.v[2 * e] = xr[e];
                    o.v[2 * e + 1] = xi[e];
                }
                stb<2 * VEC>(R.x, voff, rows.soff(j), o);
            }
        }
        return {};
    }
};

// ----------------------------------------------------------------------------------
// Adjoint of the real scan (the pages give no backward; derived from the scan form):
//   gb_t = gx_t + a_{t+1} gb_{t+1},  ga_t = gb_t x_{t-1} (x_{-1} = x0 or 0),  gx0 = a_0 gb_0.
// Backwards in time it is the real scan itself with coefficients a_{t+1} (0 after the last
// step) and inputs gx_t, so the aggregates, combine and step are RealOp's.
// ----------------------------------------------------------------------------------
struct RealBwdOp : RealOp {
    using Args = RealBwdArgs;
    static constexpr bool kReverse = true;
    template <int L>
    __device__ __forceinline__ static Chan chan(const Args&, int64_t) { return {}; }
    __device__ __forceinline__ static Agg init(const Args&, const ScanGeom&, int64_t, int64_t) { return identity(); }

    // an: a at the row above (a_{t+1}), xp: x at the row below (x_{t-1}); xshift is the
    // row's bytes when the run starts at time 0, whose x_{t-1} is x0 instead.
    struct Res { rsrc_t an, g, xp, ga, gb; unsigned xshift; int64_t T; const float* x0; const float* a0; float* gx0; };
    __device__ __forceinline__ static Res res(const Args& A, const ScanGeom& g, int64_t b, int64_t row, int64_t col0) {
        const int64_t total = g.B * g.T * g.C;
        const int64_t base = (b * g.T + row) * g.C + col0;
        const int64_t bn = base + g.C;                                           // row + 1
        const int64_t bp = (b * g.T + (row > 0 ? row - 1 : 0)) * g.C + col0;     // row - 1
        Res R;
        R.an = make_rsrc(A.a + bn, (total - bn) * 4);
        R.g = make_rsrc(A.gx + base, (total - base) * 4);
        R.xp = make_rsrc(A.x + bp, (total - bp) * 4);
        R.ga = make_rsrc(A.ga + base, (total - base) * 4);
        R.gb = make_rsrc(A.gb + base, (total - base) * 4);
        R.xshift = row > 0 ? 0u : (unsigned)(g.C * 4);
        R.T = g.T;
        R.x0 = A.x0 ? A.x0 + b * g.C + col0 : nullptr;
        R.a0 = A.a + b * g.T * g.C + col0;
        R.gx0 = A.gx0 ? A.gx0 + b * g.C + col0 : nullptr;
        return R;
    }
    template <int VEC>
    __device__ __forceinline__ static void load(const Res& R, unsigned voff, const Rows& rows, int j, In (&in)[VEC]) {
        const int64_t t = rows.t(j);
        FV<VEC> an{};
        if (t + 1 < R.T) an = ldb<VEC>(R.an, voff, rows.soff(j));
        const FV<VEC> gx = ldb<VEC>(R.g, voff, rows.soff(j));
#pragma unroll
        for (int e = 0; e < VEC; ++e) in[e] = {an.v[e], gx.v[e]};
    }
    template <int L, int VEC>
    __device__ __forceinline__ static Part run(const Res& R, const Chan (&)[VEC], const Agg (&cin)[VEC],
                               const In (&in)[L][VEC], const Local (&)[VEC], int n, unsigned voff,
                               const Rows& rows) {
        const int lane_col = (int)(voff / 4);  // this lane's first channel in the group
        FV<VEC> xp[L];
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                if (rows.t(j) > 0) {
                    xp[j] = ldb<VEC>(R.xp, voff, rows.soff(j) - R.xshift);
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) xp[j].v[e] = R.x0 ? R.x0[lane_col + e] : 0.f;
                }
            }
        }
        float s[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) s[e] = cin[e].x;
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                FV<VEC> gb, ga;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    s[e] = fmaf(in[j][e].a, s[e], in[j][e].b);
                    gb.v[e] = s[e];
                    ga.v[e] = s[e] * xp[j].v[e];
                }
                stb<VEC>(R.gb, voff, rows.soff(j), gb);
                stb<VEC>(R.ga, voff, rows.soff(j), ga);
                if (rows.t(j) == 0 && R.gx0) {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) R.gx0[lane_col + e] = R.a0[lane_col + e] * s[e];
                }
            }
        }
        return {};
    }
};

// ----------------------------------------------------------------------------------
// Adjoint of the complex scan (gradients as dL/dRe + i dL/dIm; derived from eq. lr-xx):
//   gu_t = gx_t + conj(lam) gu_{t+1},  glam = sum over batch and time of gu_t conj(x_{t-1}),
//   gx0 = conj(lam) gu_0.
// Backwards in time it is the complex scan with multiplier conj(lam), so the aggregates are
// CplxOp's.  Each slab's share of glam is a Part, summed over the slab's chunks.
// ----------------------------------------------------------------------------------
struct CplxBwdOp : CplxOp {
    using Args = CplxBwdArgs;
    static constexpr bool kReverse = true;
    static constexpr bool kParts = true;
    struct Part { double re, im; };

    template <int L>
    __device__ __forceinline__ static Chan chan(const Args& A, int64_t c) {
        Chan ch;
        ch.lr = A.lam[2 * c];
        ch.li = -A.lam[2 * c + 1];  // conj(lam)
        cpow64((double)ch.lr, (double)ch.li, L, ch.Lr, ch.Li);
        return ch;
    }
    __device__ __forceinline__ static Agg init(const Args&, const ScanGeom&, int64_t, int64_t) { return identity(); }

    struct Res { rsrc_t g, xp, gu; unsigned xshift; const float* x0; float* gx0; };
    __device__ __forceinline__ static Res res(const Args& A, const ScanGeom& g, int64_t b, int64_t row, int64_t col0) {
        const int64_t total = g.B * g.T * g.C;
        const int64_t base = (b * g.T + row) * g.C + col0;
        const int64_t bp = (b * g.T + (row > 0 ? row - 1 : 0)) * g.C + col0;
        Res R;
        R.g = make_rsrc(A.gx + 2 * base, (total - base) * 8);
        R.xp = make_rsrc(A.x + 2 * bp, (total - bp) * 8);
        R.gu = make_rsrc(A.gu + 2 * base, (total - base) * 8);
        R.xshift = row > 0 ? 0u : (unsigned)(g.C * 8);
        R.x0 = A.x0 ? A.x0 + 2 * (b * g.C + col0) : nullptr;
        R.gx0 = A.gx0 ? A.gx0 + 2 * (b * g.C + col0) : nullptr;
        return R;
    }
    template <int VEC>
    __device__ __forceinline__ static void load(const Res& R, unsigned voff, const Rows& rows, int j, In (&in)[VEC]) {
        const FV<2 * VEC> t = ldb<2 * VEC>(R.g, voff, rows.soff(j));
#pragma unroll
        for (int e = 0; e < VEC; ++e) in[e] = {t.v[2 * e], t.v[2 * e + 1]};
    }
    // Returns the lane's sum of gu_t conj(x_{t-1}) over the chunk (per channel: VEC == 1).
    template <int L, int VEC>
    __device__ __forceinline__ static Part run(const Res& R, const Chan (&ch)[VEC], const Agg (&cin)[VEC],
                               const In (&in)[L][VEC], const Local (&)[VEC], int n, unsigned voff,
                               const Rows& rows) {
        static_assert(VEC == 1, "the adjoint of the complex scan keeps one channel per lane");
        const int lane_col = (int)(voff / 8);
        FV<2> xp[L];
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                if (rows.t(j) > 0) {
                    xp[j] = ldb<2>(R.xp, voff, rows.soff(j) - R.xshift);
                } else {
                    xp[j].v[0] = R.x0 ? R.x0[2 * lane_col] : 0.f;
                    xp[j].v[1] = R.x0 ? R.x0[2 * lane_col + 1] : 0.f;
                }
            }
        }
        float sr = cin[0].xr, si = cin[0].xi, ar = 0.f, ai = 0.f;
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                const float tr = fmaf(ch[0].lr, sr, fmaf(-ch[0].li, si, in[j][0].r));
                si = fmaf(ch[0].lr, si, fmaf(ch[0].li, sr, in[j][0].i));
                sr = tr;
                FV<2> o;
                o.v[0] = sr;
                o.v[1] = si;
                stb<2>(R.gu, voff, rows.soff(j), o);
                ar = fmaf(sr, xp[j].v[0], fmaf(si, xp[j].v[1], ar));  // gu conj(x): real part
                ai = fmaf(si, xp[j].v[0], fmaf(-sr, xp[j].v[1], ai));  // imaginary part
                if (rows.t(j) == 0 && R.gx0) {
                    R.gx0[2 * lane_col] = ch[0].lr * sr - ch[0].li * si;
                    R.gx0[2 * lane_col + 1] = ch[0].lr * si + ch[0].li * sr;
                }
            }
        }
        return {(double)ar, (double)ai};
    }
};

// ----------------------------------------------------------------------------------
// Gated variants of the real scan: the coefficients a_t, b_t are formed from the gates as
// each step is loaded, so they never travel through memory (minGRU page, minGRU and minLSTM
// sections; LRU write-up, section on RWKV, for the per-channel decay).
// ----------------------------------------------------------------------------------
__device__ __forceinline__ float sigmoidf(float k) { return __builtin_amdgcn_rcpf(1.f + fast_exp2(-k * kLog2e)); }
// log(1 + e^y) without overflow: max(y, 0) + log(1 + e^{-|y|}).
__device__ __forceinline__ float softplusf(float y) {
    constexpr float kLn2 = 0.6931471805599453f;
    return fmaxf(y, 0.f) + __builtin_amdgcn_logf(1.f + fast_exp2(-fabsf(y) * kLog2e)) * kLn2;
}

// minGRU: z = sigmoid(kz), h_t = (1 - z) h_{t-1} + z h~_t.  1 - z is taken as sigmoid(-kz),
// which keeps its relative precision when z is close to 1.
struct MinGruOp : RealOp {
    using Args = MinGruArgs;
    template <int L>
    __device__ __forceinline__ static Chan chan(const Args&, int64_t) { return {}; }
    __device__ __forceinline__ static Agg init(const Args& A, const ScanGeom& g, int64_t b, int64_t c) {
        return {1.f, A.x0 ? A.x0[b * g.C + c] : 0.f};
    }
    struct Res { rsrc_t kz, h, x; };
    __device__ __forceinline__ static Res res(const Args& A, const ScanGeom& g, int64_t b, int64_t row, int64_t col0) {
        const int64_t base = (b * g.T + row) * g.C + col0, nbytes = (g.B * g.T * g.C - base) * 4;
        return {make_rsrc(A.kz + base, nbytes), make_rsrc(A.h + base, nbytes), make_rsrc(A.x + base, nbytes)};
    }
    template <int VEC>
    __device__ __forceinline__ static void load(const Res& R, unsigned voff, const Rows& rows, int j, In (&in)[VEC]) {
        const FV<VEC> k = ldb<VEC>(R.kz, voff, rows.soff(j));
        const FV<VEC> h = ldb<VEC>(R.h, voff, rows.soff(j));
#pragma unroll
        for (int e = 0; e < VEC; ++e) in[e] = {sigmoidf(-k.v[e]), sigmoidf(k.v[e]) * h.v[e]};
    }
};

// minLSTM: f = sigmoid(kf), i = sigmoid(ki), h_t = f/(f+i) h_{t-1} + i/(f+i) h~_t.  The
// normalised gates are sigmoid(+-d) with d = log f - log i = softplus(-ki) - softplus(-kf),
// which stay finite however small f and i are.
struct MinLstmOp : RealOp {
    using Args = MinLstmArgs;
    template <int L>
    __device__ __forceinline__ static Chan chan(const Args&, int64_t) { return {}; }
    __device__ __forceinline__ static Agg init(const Args& A, const ScanGeom& g, int64_t b, int64_t c) {
        return {1.f, A.x0 ? A.x0[b * g.C + c] : 0.f};
    }
    struct Res { rsrc_t kf, ki, h, x; };
    __device__ __forceinline__ static Res res(const Args& A, const ScanGeom& g, int64_t b, int64_t row, int64_t col0) {
        const int64_t base = (b * g.T + row) * g.C + col0, nbytes = (g.B * g.T * g.C - base) * 4;
        return {make_rsrc(A.kf + base, nbytes), make_rsrc(A.ki + base, nbytes), make_rsrc(A.h + base, nbytes),
                make_rsrc(A.x + base, nbytes)};
    }
    template <int VEC>
    __device__ __forceinline__ static void load(const Res& R, unsigned voff, const Rows& rows, int j, In (&in)[VEC]) {
        const FV<VEC> kf = ldb<VEC>(R.kf, voff, rows.soff(j));
        const FV<VEC> ki = ldb<VEC>(R.ki, voff, rows.soff(j));
        const FV<VEC> h = ldb<VEC>(R.h, voff, rows.soff(j));
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float d = softplusf(-ki.v[e]) - softplusf(-kf.v[e]);
            in[e] = {sigmoidf(d), sigmoidf(-d) * h.v[e]};
        }
    }
};

// One decay per channel: x_t = lam_c x_{t-1} + u_t (an SLRU).  The decay lives in the
// channel constants, so only u is streamed.
struct RealDecayOp {
    using Args = RealDecayArgs;
    static constexpr bool kReverse = false;
    static constexpr bool kParts = false;
    using Part = NoPart;
    template <class AnyArgs, class AnyAgg>
    __device__ __forceinline__ static void finish(const AnyArgs&, const ScanGeom&, int64_t, int64_t, const AnyAgg&) {}
    struct Chan { float lam; };
    struct In { float u; };
    struct Local {};
    struct Agg { float m, x; };

    template <int L>
    __device__ __forceinline__ static Chan chan(const Args& A, int64_t c) { return {A.lam[c]}; }
    __device__ __forceinline__ static Agg identity() { return {1.f, 0.f}; }
    __device__ __forceinline__ static Agg init(const Args& A, const ScanGeom& g, int64_t b, int64_t c) {
        return {1.f, A.x0 ? A.x0[b * g.C + c] : 0.f};
    }
    static constexpr int kFloats = 1;
    struct Res { rsrc_t u, x; };
    __device__ __forceinline__ static Res res(const Args& A, const ScanGeom& g, int64_t b, int64_t row, int64_t col0) {
        const int64_t base = (b * g.T + row) * g.C + col0, nbytes = (g.B * g.T * g.C - base) * 4;
        return {make_rsrc(A.u + base, nbytes), make_rsrc(A.x + base, nbytes)};
    }
    template <int VEC>
    __device__ __forceinline__ static void load(const Res& R, unsigned voff, const Rows& rows, int j, In (&in)[VEC]) {
        const FV<VEC> u = ldb<VEC>(R.u, voff, rows.soff(j));
#pragma unroll
        for (int e = 0; e < VEC; ++e) in[e] = {u.v[e]};
    }
    template <int VEC>
    __device__ __forceinline__ static void zero(In (&in)[VEC]) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) in[e] = {0.f};
    }
    template <int L, int VEC>
    __device__ __forceinline__ static Agg reduce(const Chan& ch, In (&in)[L][VEC], int e, int n, Local&) {
        float m = 1.f, x = 0.f;
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                x = fmaf(ch.lam, x, in[j][e].u);
                m *= ch.lam;
            }
        }
        return {m, x};
    }
    __device__ __forceinline__ static Agg combine(const Chan&, const Agg& s1, const Agg& s2, int64_t) {
        return {s1.m * s2.m, fmaf(s2.m, s1.x, s2.x)};
    }
    __device__ __forceinline__ static Agg step(const Chan& ch, const Agg& s, const In& x) {
        return {s.m * ch.lam, fmaf(ch.lam, s.x, x.u)};
    }
    template <int L, int VEC>
    __device__ __forceinline__ static Part run(const Res& R, const Chan (&ch)[VEC], const Agg (&cin)[VEC],
                                               const In (&in)[L][VEC], const Local (&)[VEC], int n, unsigned voff,
                                               const Rows& rows) {
        float x[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[e] = cin[e].x;
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                FV<VEC> o;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    x[e] = fmaf(ch[e].lam, x[e], in[j][e].u);
                    o.v[e] = x[e];
                }
                stb<VEC>(R.x, voff, rows.soff(j), o);
            }
        }
        return {};
    }
};

// The LRU with normalised input (LRU write-up, initialisation section):
// x_t = lam x_{t-1} + gamma u_t, gamma = sqrt(1 - |lam|^2) per channel.  The loaded inputs
// are scaled once, when the chunk is reduced (the re-run then uses them as they are), and
// in the look-back's per-step recompute.
struct CplxNormOp : CplxOp {
    struct Chan : CplxOp::Chan { float gamma; };
    template <int L>
    __device__ __forceinline__ static Chan chan(const Args& A, int64_t c) {
        Chan ch;
        static_cast<CplxOp::Chan&>(ch) = CplxOp::template chan<L>(A, c);
        const double lr = ch.lr, li = ch.li;
        ch.gamma = (float)sqrt(fmax(0.0, 1.0 - (lr * lr + li * li)));
        return ch;
    }
    template <int L, int VEC>
    __device__ __forceinline__ static Agg reduce(const Chan& ch, In (&in)[L][VEC], int e, int n, Local& loc) {
#pragma unroll
        for (int j = 0; j < L; ++j) in[j][e] = {ch.gamma * in[j][e].r, ch.gamma * in[j][e].i};
        return CplxOp::template reduce<L, VEC>(ch, in, e, n, loc);
    }
    __device__ __forceinline__ static Agg step(const Chan& ch, const Agg& s, const In& x) {
        return CplxOp::step(ch, s, In{ch.gamma * x.r, ch.gamma * x.i});
    }
    template <int L, int VEC>
    __device__ __forceinline__ static Part run(const Res& R, const Chan (&ch)[VEC], const Agg (&cin)[VEC],
                                               const In (&in)[L][VEC], const Local (&loc)[VEC], int n, unsigned voff,
                                               const Rows& rows) {
        CplxOp::Chan cb[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) cb[e] = ch[e];
        return CplxOp::template run<L, VEC>(R, cb, cin, in, loc, n, voff, rows);
    }
};

// ----------------------------------------------------------------------------------
// Adjoints of the gated variants (chain rule of the forward readings; the pages give no
// backward).  Backwards in time each is the real (or complex) scan's adjoint whose
// multiplier is formed from the gates as the step is loaded; the step's own gate
// derivatives are taken where the adjoint state d_t is formed, with h_{t-1} read from the
// forward output (x0 at t = 0).
// ----------------------------------------------------------------------------------

// Buffers shared by the real adjoints: the row above (t+1) of the multiplier's inputs, the
// row itself, the row below of x.  xshift as in RealBwdOp.
struct BwdRows {
    __device__ __forceinline__ static int64_t above(const ScanGeom& g, int64_t base) { return base + g.C; }
    __device__ __forceinline__ static int64_t below(const ScanGeom& g, int64_t b, int64_t row, int64_t col0) {
        return (b * g.T + (row > 0 ? row - 1 : 0)) * g.C + col0;
    }
};

// sigma(k) and sigma(-k) from one exponential: with e = e^{-|k|}, sigma(|k|) = 1/(1+e) and
// sigma(-|k|) = e/(1+e), both without cancellation.
__device__ __forceinline__ void sigmoid_pair(float k, float& s, float& sc) {
    const float e = fast_exp2(-fabsf(k) * kLog2e);
    const float r = __builtin_amdgcn_rcpf(1.f + e);
    const float q = e * r;
    s = k >= 0.f ? r : q;
    sc = k >= 0.f ? q : r;
}
__device__ __forceinline__ float sigmoid_neg(float k) {
    float s, sc;
    sigmoid_pair(k, s, sc);
    return sc;
}

// The gated adjoints keep the RAW gate logits of row t+1 in their chunk registers (not the
// multiplier formed from them): step j's multiplier needs row t+1 and its own derivatives
// need row t, which is step j+1's row t+1, so each gate row is read from memory once (one
// extra row per chunk).  Past the last row the logits take values whose multiplier is 0
// (minGRU: k_z = +inf; minLSTM: k_f = -inf, a closed forget gate).

// minGRU: d_t = gx_t + sigmoid(-kz_{t+1}) d_{t+1};  dL/dkz_t = d_t z_t (1 - z_t) (h~_t - h_{t-1}),
// dL/dh~_t = d_t z_t, dL/dx0 = (1 - z_0) d_0.
struct MinGruBwdOp : RealOp {
    using Args = MinGruBwdArgs;
    static constexpr bool kReverse = true;
    struct In { float k, g; };  // kz_{t+1} (+inf past the end), gx_t
    template <int L>
    __device__ __forceinline__ static Chan chan(const Args&, int64_t) { return {}; }
    __device__ __forceinline__ static Agg init(const Args&, const ScanGeom&, int64_t, int64_t) { return identity(); }

    struct Res { rsrc_t kn, g, k, h, xp, gk, gh; unsigned xshift; int64_t T; const float* x0; float* gx0; };
    __device__ __forceinline__ static Res res(const Args& A, const ScanGeom& g, int64_t b, int64_t row, int64_t col0) {
        const int64_t total = g.B * g.T * g.C;
        const int64_t base = (b * g.T + row) * g.C + col0;
        const int64_t bn = BwdRows::above(g, base), bp = BwdRows::below(g, b, row, col0);
        Res R;
        R.kn = make_rsrc(A.kz + bn, (total - bn) * 4);
        R.g = make_rsrc(A.gx + base, (total - base) * 4);
        R.k = make_rsrc(A.kz + base, (total - base) * 4);
        R.h = make_rsrc(A.h + base, (total - base) * 4);
        R.xp = make_rsrc(A.x + bp, (total - bp) * 4);
        R.gk = make_rsrc(A.gkz + base, (total - base) * 4);
        R.gh = make_rsrc(A.gh + base, (total - base) * 4);
        R.xshift = row > 0 ? 0u : (unsigned)(g.C * 4);
        R.T = g.T;
        R.x0 = A.x0 ? A.x0 + b * g.C + col0 : nullptr;
        R.gx0 = A.gx0 ? A.gx0 + b * g.C + col0 : nullptr;
        return R;
    }
    template <int VEC>
    __device__ __forceinline__ static void load(const Res& R, unsigned voff, const Rows& rows, int j, In (&in)[VEC]) {
        const bool last = rows.t(j) + 1 >= R.T;
        FV<VEC> kn{};
        if (!last) kn = ldb<VEC>(R.kn, voff, rows.soff(j));
        const FV<VEC> gx = ldb<VEC>(R.g, voff, rows.soff(j));
#pragma unroll
        for (int e = 0; e < VEC; ++e) in[e] = {last ? __builtin_inff() : kn.v[e], gx.v[e]};
    }
    template <int VEC>
    __device__ __forceinline__ static void zero(In (&in)[VEC]) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) in[e] = {__builtin_inff(), 0.f};
    }
    template <int L, int VEC>
    __device__ __forceinline__ static Agg reduce(const Chan&, In (&in)[L][VEC], int e, int n, Local&) {
        float m = 1.f, x = 0.f;
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                const float a = sigmoid_neg(in[j][e].k);
                x = fmaf(a, x, in[j][e].g);
                m *= a;
            }
        }
        return {m, x};
    }
    __device__ __forceinline__ static Agg step(const Chan&, const Agg& s, const In& x) {
        const float a = sigmoid_neg(x.k);
        return {s.m * a, fmaf(a, s.x, x.g)};
    }
    template <int L, int VEC>
    __device__ __forceinline__ static Part run(const Res& R, const Chan (&)[VEC], const Agg (&cin)[VEC],
                                               const In (&in)[L][VEC], const Local (&)[VEC], int n, unsigned voff,
                                               const Rows& rows) {
        static_assert(VEC == 1, "the adjoints keep one channel per lane");
        const int lane_col = (int)(voff / 4);
        float xp[L], hh[L];
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                xp[j] = rows.t(j) > 0 ? ldb<1>(R.xp, voff, rows.soff(j) - R.xshift).v[0]
                                      : (R.x0 ? R.x0[lane_col] : 0.f);
                hh[j] = ldb<1>(R.h, voff, rows.soff(j)).v[0];
            }
        }
        // The gate row of the chunk's earliest step (the only one not among the k_{t+1}).
        const float k_low = n > 0 ? ldb<1>(R.k, voff, rows.soff(n - 1)).v[0] : 0.f;
        float d = cin[0].x, a = sigmoid_neg(in[0][0].k);
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                d = fmaf(a, d, in[j][0].g);
                const float kz = (j + 1 < L && j + 1 < n) ? in[j + 1 < L ? j + 1 : j][0].k : k_low;
                float z, zc;
                sigmoid_pair(kz, z, zc);
                FV<1> gk, gh;
                gk.v[0] = d * (z * zc) * (hh[j] - xp[j]);
                gh.v[0] = d * z;
                stb<1>(R.gk, voff, rows.soff(j), gk);
                stb<1>(R.gh, voff, rows.soff(j), gh);
                if (rows.t(j) == 0 && R.gx0) R.gx0[lane_col] = zc * d;
                a = zc;  // the multiplier of the next step (one time step earlier)
            }
        }
        return {};
    }
};

// minLSTM: with a = sigmoid(dd), dd = softplus(-ki) - softplus(-kf) (the weight f/(f+i) of
// h_{t-1}), d_t = gx_t + a_{t+1} d_{t+1};  g_dd = a (1 - a) d_t (h_{t-1} - h~_t),
// dL/dkf = g_dd sigmoid(-kf), dL/dki = -g_dd sigmoid(-ki), dL/dh~_t = d_t (1 - a_t),
// dL/dx0 = a_0 d_0.
struct MinLstmBwdOp : RealOp {
    using Args = MinLstmBwdArgs;
    static constexpr bool kReverse = true;
    struct In { float f, i, g; };  // kf_{t+1} (-inf past the end), ki_{t+1}, gx_t
    template <int L>
    __device__ __forceinline__ static Chan chan(const Args&, int64_t) { return {}; }
    __device__ __forceinline__ static Agg init(const Args&, const ScanGeom&, int64_t, int64_t) { return identity(); }

    struct Res { rsrc_t fn, in_, g, f, i, h, xp, gf, gi, gh; unsigned xshift; int64_t T; const float* x0; float* gx0; };
    __device__ __forceinline__ static Res res(const Args& A, const ScanGeom& g, int64_t b, int64_t row, int64_t col0) {
        const int64_t total = g.B * g.T * g.C;
        const int64_t base = (b * g.T + row) * g.C + col0;
        const int64_t bn = BwdRows::above(g, base), bp = BwdRows::below(g, b, row, col0);
        Res R;
        R.fn = make_rsrc(A.kf + bn, (total - bn) * 4);
        R.in_ = make_rsrc(A.ki + bn, (total - bn) * 4);
        R.g = make_rsrc(A.gx + base, (total - base) * 4);
        R.f = make_rsrc(A.kf + base, (total - base) * 4);
        R.i = make_rsrc(A.ki + base, (total - base) * 4);
        R.h = make_rsrc(A.h + base, (total - base) * 4);
        R.xp = make_rsrc(A.x + bp, (total - bp) * 4);
        R.gf = make_rsrc(A.gkf + base, (total - base) * 4);
        R.gi = make_rsrc(A.gki + base, (total - base) * 4);
        R.gh = make_rsrc(A.gh + base, (total - base) * 4);
        R.xshift = row > 0 ? 0u : (unsigned)(g.C * 4);
        R.T = g.T;
        R.x0 = A.x0 ? A.x0 + b * g.C + col0 : nullptr;
        R.gx0 = A.gx0 ? A.gx0 + b * g.C + col0 : nullptr;
        return R;
    }
    __device__ __forceinline__ static float logit(float kf, float ki) { return softplusf(-ki) - softplusf(-kf); }
    template <int VEC>
    __device__ __forceinline__ static void load(const Res& R, unsigned voff, const Rows& rows, int j, In (&in)[VEC]) {
        const bool last = rows.t(j) + 1 >= R.T;
        FV<VEC> fn{}, inn{};
        if (!last) {
            fn = ldb<VEC>(R.fn, voff, rows.soff(j));
            inn = ldb<VEC>(R.in_, voff, rows.soff(j));
        }
        const FV<VEC> gx = ldb<VEC>(R.g, voff, rows.soff(j));
#pragma unroll
        for (int e = 0; e < VEC; ++e) in[e] = {last ? -__builtin_inff() : fn.v[e], inn.v[e], gx.v[e]};
    }
    template <int VEC>
    __device__ __forceinline__ static void zero(In (&in)[VEC]) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) in[e] = {-__builtin_inff(), 0.f, 0.f};
    }
    // The multiplier a = f/(f+i) of the step whose gate logits are (kf, ki); 0 for kf = -inf.
    __device__ __forceinline__ static float mult(float kf, float ki) {
        float a, ac;
        sigmoid_pair(logit(kf, ki), a, ac);
        return a;
    }
    template <int L, int VEC>
    __device__ __forceinline__ static Agg reduce(const Chan&, In (&in)[L][VEC], int e, int n, Local&) {
        float m = 1.f, x = 0.f;
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                const float a = mult(in[j][e].f, in[j][e].i);
                x = fmaf(a, x, in[j][e].g);
                m *= a;
            }
        }
        return {m, x};
    }
    __device__ __forceinline__ static Agg step(const Chan&, const Agg& s, const In& x) {
        const float a = mult(x.f, x.i);
        return {s.m * a, fmaf(a, s.x, x.g)};
    }
    template <int L, int VEC>
    __device__ __forceinline__ static Part run(const Res& R, const Chan (&)[VEC], const Agg (&cin)[VEC],
                                               const In (&in)[L][VEC], const Local (&)[VEC], int n, unsigned voff,
                                               const Rows& rows) {
        static_assert(VEC == 1, "the adjoints keep one channel per lane");
        const int lane_col = (int)(voff / 4);
        float xp[L], hh[L];
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                xp[j] = rows.t(j) > 0 ? ldb<1>(R.xp, voff, rows.soff(j) - R.xshift).v[0]
                                      : (R.x0 ? R.x0[lane_col] : 0.f);
                hh[j] = ldb<1>(R.h, voff, rows.soff(j)).v[0];
            }
        }
        const float f_low = n > 0 ? ldb<1>(R.f, voff, rows.soff(n - 1)).v[0] : 0.f;
        const float i_low = n > 0 ? ldb<1>(R.i, voff, rows.soff(n - 1)).v[0] : 0.f;
        float d = cin[0].x, a = mult(in[0][0].f, in[0][0].i);
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                d = fmaf(a, d, in[j][0].g);
                const bool inner = j + 1 < L && j + 1 < n;
                const int jn = j + 1 < L ? j + 1 : j;
                const float kf = inner ? in[jn][0].f : f_low, ki = inner ? in[jn][0].i : i_low;
                float at, ac, sf, sfc, si, sic;
                sigmoid_pair(softplusf(-ki) - softplusf(-kf), at, ac);
                sigmoid_pair(kf, sf, sfc);
                sigmoid_pair(ki, si, sic);
                const float gdd = (at * ac) * d * (xp[j] - hh[j]);
                FV<1> gf, gi, gh;
                gf.v[0] = gdd * sfc;
                gi.v[0] = -gdd * sic;
                gh.v[0] = d * ac;
                stb<1>(R.gf, voff, rows.soff(j), gf);
                stb<1>(R.gi, voff, rows.soff(j), gi);
                stb<1>(R.gh, voff, rows.soff(j), gh);
                if (rows.t(j) == 0 && R.gx0) R.gx0[lane_col] = at * d;
                a = at;
            }
        }
        return {};
    }
};

// The per-channel decay: d_t = gx_t + lam d_{t+1};  dL/du_t = d_t, dL/dlam = sum over batch
// and time of d_t x_{t-1} (a per-slab share, summed like the complex adjoint's),
// dL/dx0 = lam d_0.
struct RealDecayBwdOp : RealDecayOp {
    using Args = RealDecayBwdArgs;
    static constexpr bool kReverse = true;
    static constexpr bool kParts = true;
    struct Part { double re, im; };
    template <int L>
    __device__ __forceinline__ static Chan chan(const Args& A, int64_t c) { return {A.lam[c]}; }
    __device__ __forceinline__ static Agg init(const Args&, const ScanGeom&, int64_t, int64_t) { return identity(); }

    struct Res { rsrc_t g, xp, gu; unsigned xshift; const float* x0; float* gx0; };
    __device__ __forceinline__ static Res res(const Args& A, const ScanGeom& g, int64_t b, int64_t row, int64_t col0) {
        const int64_t total = g.B * g.T * g.C;
        const int64_t base = (b * g.T + row) * g.C + col0, bp = BwdRows::below(g, b, row, col0);
        Res R;
        R.g = make_rsrc(A.gx + base, (total - base) * 4);
        R.xp = make_rsrc(A.x + bp, (total - bp) * 4);
        R.gu = make_rsrc(A.gu + base, (total - base) * 4);
        R.xshift = row > 0 ? 0u : (unsigned)(g.C * 4);
        R.x0 = A.x0 ? A.x0 + b * g.C + col0 : nullptr;
        R.gx0 = A.gx0 ? A.gx0 + b * g.C + col0 : nullptr;
        return R;
    }
    template <int VEC>
    __device__ __forceinline__ static void load(const Res& R, unsigned voff, const Rows& rows, int j, In (&in)[VEC]) {
        const FV<VEC> gx = ldb<VEC>(R.g, voff, rows.soff(j));
#pragma unroll
        for (int e = 0; e < VEC; ++e) in[e] = {gx.v[e]};
    }
    template <int L, int VEC>
    __device__ __forceinline__ static Part run(const Res& R, const Chan (&ch)[VEC], const Agg (&cin)[VEC],
                                               const In (&in)[L][VEC], const Local (&)[VEC], int n, unsigned voff,
                                               const Rows& rows) {
        static_assert(VEC == 1, "the adjoints keep one channel per lane");
        const int lane_col = (int)(voff / 4);
        float xp[L];
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                xp[j] = rows.t(j) > 0 ? ldb<1>(R.xp, voff, rows.soff(j) - R.xshift).v[0]
                                      : (R.x0 ? R.x0[lane_col] : 0.f);
            }
        }
        float d = cin[0].x, acc = 0.f;
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                d = fmaf(ch[0].lam, d, in[j][0].u);
                FV<1> o;
                o.v[0] = d;
                stb<1>(R.gu, voff, rows.soff(j), o);
                acc = fmaf(d, xp[j], acc);
                if (rows.t(j) == 0 && R.gx0) R.gx0[lane_col] = ch[0].lam * d;
            }
        }
        return {(double)acc, 0.0};
    }
};

// The normalised LRU: s_t = gx_t + conj(lam) s_{t+1};  dL/du_t = gamma s_t,
// dL/dx0 = conj(lam) s_0, and dL/dlam = sum of s_t conj(x_{t-1}) + kg Re(conj(s_t) u_t) with
// kg = -lam / gamma (dgamma/dRe + i dgamma/dIm, times 1/dL/dgamma's own sum), 0 where gamma = 0.
struct CplxNormBwdOp : CplxBwdOp {
    struct Chan : CplxBwdOp::Chan { float gamma, kgr, kgi; };
    template <int L>
    __device__ __forceinline__ static Chan chan(const Args& A, int64_t c) {
        Chan ch;
        static_cast<CplxBwdOp::Chan&>(ch) = CplxBwdOp::template chan<L>(A, c);
        const double lr = A.lam[2 * c], li = A.lam[2 * c + 1];
        const double gam = sqrt(fmax(0.0, 1.0 - (lr * lr + li * li)));
        ch.gamma = (float)gam;
        ch.kgr = gam > 0.0 ? (float)(-lr / gam) : 0.f;
        ch.kgi = gam > 0.0 ? (float)(-li / gam) : 0.f;
        return ch;
    }
    struct Res : CplxBwdOp::Res { rsrc_t u; };
    __device__ __forceinline__ static Res res(const Args& A, const ScanGeom& g, int64_t b, int64_t row, int64_t col0) {
        Res R;
        static_cast<CplxBwdOp::Res&>(R) = CplxBwdOp::res(A, g, b, row, col0);
        const int64_t total = g.B * g.T * g.C;
        const int64_t base = (b * g.T + row) * g.C + col0;
        R.u = make_rsrc(A.u + 2 * base, (total - base) * 8);
        return R;
    }
    template <int L, int VEC>
    __device__ __forceinline__ static Part run(const Res& R, const Chan (&ch)[VEC], const Agg (&cin)[VEC],
                                               const In (&in)[L][VEC], const Local (&)[VEC], int n, unsigned voff,
                                               const Rows& rows) {
        static_assert(VEC == 1, "the adjoint of the complex scan keeps one channel per lane");
        const int lane_col = (int)(voff / 8);
        FV<2> xp[L], uu[L];
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                if (rows.t(j) > 0) {
                    xp[j] = ldb<2>(R.xp, voff, rows.soff(j) - R.xshift);
                } else {
                    xp[j].v[0] = R.x0 ? R.x0[2 * lane_col] : 0.f;
                    xp[j].v[1] = R.x0 ? R.x0[2 * lane_col + 1] : 0.f;
                }
                uu[j] = ldb<2>(R.u, voff, rows.soff(j));
            }
        }
        float sr = cin[0].xr, si = cin[0].xi, ar = 0.f, ai = 0.f, dg = 0.f;
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                const float tr = fmaf(ch[0].lr, sr, fmaf(-ch[0].li, si, in[j][0].r));
                si = fmaf(ch[0].lr, si, fmaf(ch[0].li, sr, in[j][0].i));
                sr = tr;
                FV<2> o;
                o.v[0] = ch[0].gamma * sr;
                o.v[1] = ch[0].gamma * si;
                stb<2>(R.gu, voff, rows.soff(j), o);
                ar = fmaf(sr, xp[j].v[0], fmaf(si, xp[j].v[1], ar));  // s conj(x): real part
                ai = fmaf(si, xp[j].v[0], fmaf(-sr, xp[j].v[1], ai));  // imaginary part
                dg = fmaf(sr, uu[j].v[0], fmaf(si, uu[j].v[1], dg));   // Re(conj(s) u)
                if (rows.t(j) == 0 && R.gx0) {
                    R.gx0[2 * lane_col] = ch[0].lr * sr - ch[0].li * si;
                    R.gx0[2 * lane_col + 1] = ch[0].lr * si + ch[0].li * sr;
                }
            }
        }
        return {(double)fmaf(ch[0].kgr, dg, ar), (double)fmaf(ch[0].kgi, dg, ai)};
    }
};

}  // namespace linrec

// wkv_ckpt.hip -- the checkpointing WKV-4 forward on gfx950: y of eq. (14) (RWKV-LLM page,
// "Time-mixing block"), and on the way the forward sums (A, B, A', B') at the end of every
// slab of the backward's gradient kernel (every 56 steps), so that a training step's backward
// can skip its own forward pass over k and v (the state kernel).
//
// It is the chunked look-back scan of the plain forward (one channel per lane, slabs of 8
// chunks of 16 steps) with a wider aggregate: the chunk reduction also forms A' and B' (each
// weight times its distance to the chunk end), and slabs combine with the float64 fold of
// wkv_sums.hpp.  Each chunk starts its re-run from its carry-in, the sums before its first
// step.  A chunk that contains a multiple of 56 (at most one: 16 < 56) forms the sums there
// -- the carry-in followed by the steps before it, from the chunk's own weights (or, behind a
// spike that may have flushed them, from k and v step by step) -- and writes them in the
// record layout the gradient kernel reads.  The re-run itself is the plain
// forward's (A and B rounded to float32 at the carry-in), gated by sigma(r) when r is given.
// A carried state seeds the chain (the slab-0 carry) and the last slab writes the final state.
#include "scan_kernel.hpp"
#include "wkv_backward.hpp"
#include "wkv_sums.hpp"

namespace linrec {

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kCkptSlab = 56;  // steps between kept sums: the gradient kernel's slab (7 x 8)

struct WkvCkptArgs : WkvArgs {
    uint32_t* ckpt;  // (B*ngrp, nck, 5 dwords, 64 lanes) kept sums (FwdRec)
    int64_t nck;     // records per channel group: ceil(T / 56)
};

// The sums s1, then a span of n2 steps whose sums (a, b, ad, bd) carry the exponent p2 + ne om
// (not an integer): as fwd_combine, with that exponent kept split (p2 and the resulting
// exponent are integers, ne om = hi + lo exactly), so the scale factors lose nothing to its
// rounding.
__device__ __forceinline__ Fwd fwd_combine_shifted(float om, const Fwd& s1, float a, float b, float ad, float bd,
                                                   float p2, int ne, int n2) {
    const Split d = mul_split((float)n2, om), e = mul_split((float)ne, om);
    const float P = ceilf(fmaxf(mag(s1.p, (float)s1.b) - d.hi, mag(p2 + e.hi, b)));
    const double f1 = fast_exp2(((s1.p - P) - d.hi) - d.lo);
    const double f2 = fast_exp2(((p2 - P) + e.hi) + e.lo);
    const double fn = (double)n2;
    return {fma(s1.a, f1, a * f2), fma(s1.b, f1, b * f2), fma(fma(fn, s1.a, s1.ad), f1, ad * f2),
            fma(fma(fn, s1.b, s1.bd), f1, bd * f2), P};
}

// GATED: the output is sigma(r) wkv (eq. (15)).  STATE: the sequence starts from a carried
// state s_in (the past sums (a, b, p) of every earlier token, as wkv4_forward_ex takes it),
// whose own derivatives in w are zero (the state is an input: its gradient is dL/d(a, b)),
// and the state after the last token is written to s_out.  The plain instance compiles none
// of either.
template <bool GATED, bool STATE>
struct WkvCkptOpT {
    using Args = WkvCkptArgs;
    using Base = typename std::conditional<GATED || STATE, WkvExtOp, WkvOp>::type;
    static constexpr bool kReverse = false;
    static constexpr bool kParts = false;
    static constexpr bool kChanLate = true;  // w, u are read after the chunk's loads are issued
    using Part = NoPart;
    using Chan = typename Base::Chan;
    using In = typename Base::In;
    using Local = typename Base::Local;
    using Agg = Fwd;
    static constexpr int kFloats = 1;
    // The plain buffers, and where the run starting at `row` keeps sums: at step js of the
    // run (the first multiple of 56 at or after row, if before T), into record m.
    struct Res {
        typename Base::Res base;
        uint32_t* rec;
        int64_t m;
        int js;
    };

    template <int L>
    __device__ __forceinline__ static Chan chan(const Args& A, int64_t c) { return Base::template chan<L>(A, c); }
    __device__ __forceinline__ static Agg identity() { return fwd_identity(); }
    // The sums before the first token: empty, or the carried state in base-2 form (A' = B' = 0).
    __device__ __forceinline__ static Agg init(const Args& A, const ScanGeom& g, int64_t b, int64_t c) {
        if constexpr (STATE) {
            if (A.s_in) {
                const float* s = A.s_in + 3 * (b * g.C + c);
                const Base2State x = state_from_natural(s[0], s[1], s[2]);
                if (x.a != 0.f || x.b != 0.f) return {(double)x.a, (double)x.b, 0.0, 0.0, x.p};
            }
        }
        return fwd_identity();
    }
    // The state after the last token, as wkv4_forward_ex writes it.
    __device__ __forceinline__ static void finish(const Args& A, const ScanGeom& g, int64_t b, int64_t c,
                                                  const Agg& s) {
        if constexpr (STATE) {
            if (!A.s_out) return;
            float* o = A.s_out + 3 * (b * g.C + c);
            state_to_natural({(float)s.a, (float)s.b, s.p}, o[0], o[1], o[2]);
        }
    }
    __device__ __forceinline__ static Res res(const Args& A, const ScanGeom& g, int64_t b, int64_t row, int64_t col0) {
        Res R;
        R.base = Base::res(A, g, b, row, col0);
        const int64_t mb = row > 0 ? ((row + kCkptSlab - 1) / kCkptSlab) * kCkptSlab : kCkptSlab;
        R.js = (mb < g.T) ? (int)(mb - row) : -1;
        R.m = mb / kCkptSlab - 1;
        R.rec = A.ckpt + (b * g.ngrp + col0 / 64) * A.nck * (64 * kDwords<FwdRec>);
        return R;
    }
    template <int VEC>
    __device__ __forceinline__ static void load(const Res& R, unsigned voff, const Rows& rows, int j, In (&in)[VEC]) {
        Base::template load<VEC>(R.base, voff, rows, j, in);
    }
    template <int VEC>
    __device__ __forceinline__ static void zero(In (&in)[VEC]) {
        Base::template zero<VEC>(in);
    }

    // The plain reduction (weights g_j = 2^{m_j - p} kept in kk for the re-run), plus A' and B'
    // with step j weighted by its distance n-1-j to the chunk end.
    template <int L, int VEC>
    __device__ __forceinline__ static Agg reduce(const Chan& ch, In (&in)[L][VEC], int e, int n, Local& loc) {
        if (n <= 0) {
            loc = {kEmpty, kEmpty};
            return fwd_identity();
        }
        float m[L];
        float mx = kEmpty;
#pragma unroll
        for (int j = 0; j < L; ++j) {
            m[j] = (j < n) ? fmaf(-(float)(n - 1 - j), ch.om, in[j][e].kk) : kEmpty;
            mx = fmaxf(mx, m[j]);
        }
        const float p = ceilf(mx);
        float a = 0.f, b = 0.f, ad = 0.f, bd = 0.f;
#pragma unroll
        for (int j = 0; j < L; ++j) {
            const float gj = fast_exp2(m[j] - p);  // 0 for the unused slots
            in[j][e].kk = gj;
            const float fd = gj * (float)max(n - 1 - j, 0);
            a = fmaf(gj, in[j][e].v, a);
            b += gj;
            ad = fmaf(fd, in[j][e].v, ad);
            bd += fd;
        }
        loc = {p, m[0] - p};
        return {a, b, ad, bd, p};
    }

    __device__ __forceinline__ static Agg combine(const Chan& ch, const Agg& s1, const Agg& s2, int64_t n2) {
        return fwd_combine(ch.om, s1, s2, n2);
    }
    __device__ __forceinline__ static Agg step(const Chan& ch, const Agg& s, const In& x) {
        Fwd t = s;
        fwd_advance(ch.om, t, x.kk, (double)x.v, mag(s.p, (float)s.b));
        return t;
    }

    template <int L, int VEC>
    __device__ __forceinline__ static Part run(const Res& R, const Chan (&ch)[VEC], const Agg (&cin)[VEC],
                                               const In (&in)[L][VEC], const Local (&loc)[VEC], int n, unsigned voff,
                                               const Rows& rows) {
        static_assert(VEC == 1, "the kept sums are laid out for one channel per lane");
        if (R.js >= 0 && R.js < n) {  // a multiple of 56 falls in this chunk (same for the wave)
            // The sums before step js: the carry-in followed by steps 0 .. js-1.  Their weights
            // at js are the chunk's g_j (relative to its end, exponent p) times 2^{(n-js) om}.
            // If a later step of the chunk dominates so much that these g_j may have lost
            // terms to underflow, the steps are re-read and advanced exactly instead.
            Fwd st = cin[0];
            const int js = R.js;
            if (js > 0) {
                float a = 0.f, b = 0.f, ad = 0.f, bd = 0.f, gmax = 0.f;
#pragma unroll
                for (int j = 0; j < L; ++j) {
                    if (j < js) {
                        const float gj = in[j][0].kk, fd = gj * (float)(js - 1 - j);
                        a = fmaf(gj, in[j][0].v, a);
                        b += gj;
                        ad = fmaf(fd, in[j][0].v, ad);
                        bd += fd;
                        gmax = fmaxf(gmax, gj);
                    }
                }
                if (gmax >= 0x1p-60f) {
                    st = fwd_combine_shifted(ch[0].om, st, a, b, ad, bd, loc[0].p, n - js, js);
                } else {
#pragma unroll
                    for (int j = 0; j < L; ++j) {
                        if (j < js) {
                            const float kk = ldb<1>(R.base.k, voff, rows.soff(j)).v[0] * kLog2e;
                            fwd_advance(ch[0].om, st, kk, (double)in[j][0].v, mag(st.p, (float)st.b));
                        }
                    }
                }
            }
            // This lane's entry of the kept sums.  A lane past the last channel runs the
            // chunk too (its buffer offset out of range: loads 0, stores dropped) but keeps
            // nothing: its offset names no entry.
            const unsigned slot = voff >> 2;
            if (slot < 64) {
                const FwdRec x[1] = {fwd_to_rec(st)};
                store_record<1>(R.rec, R.m, (int)slot, x);
            }
        }
        typename Base::Agg c[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) c[e] = {(float)cin[e].a, (float)cin[e].b, cin[e].p};
        return Base::template run<L, VEC>(R.base, ch, c, in, loc, n, voff, rows);
    }
};

}  // namespace

// The gated instance also holds r per step: at 6 waves per SIMD (80 VGPRs) it spills around
// the kept sums; 5 (96 VGPRs) does not, and measured faster (gated step 984 -> 948 us).  The
// carried-state instances share the gated one's per-step inputs (r is loaded when given).
namespace scan_kernel {
template <>
constexpr int scan_waves_per_eu<WkvCkptOpT<true, false>, 1, 16>() {
    return 5;
}
template <>
constexpr int scan_waves_per_eu<WkvCkptOpT<false, true>, 1, 16>() {
    return 5;
}
template <>
constexpr int scan_waves_per_eu<WkvCkptOpT<true, true>, 1, 16>() {
    return 5;
}
}  // namespace scan_kernel

// Slabs of the forward: 8 chunks of 16 steps.
constexpr int kCkptNW = 8, kCkptL = 16;

size_t wkv_ckpt_bytes(int64_t B, int64_t T, int64_t C) {
    const int64_t nck = (T + kCkptSlab - 1) / kCkptSlab;
    return (size_t)(B * ((C + 63) / 64) * nck * 64) * sizeof(FwdRec);
}

size_t wkv_ckpt_forward_ws_bytes(int64_t B, int64_t T, int64_t C) {
    const int64_t nslab = (T + kCkptNW * kCkptL - 1) / (kCkptNW * kCkptL);
    if (nslab <= 1) return 0;
    const int64_t nwg = B * ((C + 63) / 64) * nslab;
    return align256((size_t)nwg * 8) + 2 * align256((size_t)(nwg * 64) * sizeof(RecordOf<Fwd>::type));
}

hipError_t run_wkv_forward_ckpt(const WkvArgs& A, int64_t B, int64_t T, int64_t C, void* ckpt, void* ws,
                                uint64_t tag, int spin, bool sep, hipStream_t st) {
    // The kept sums are the gradient kernel's slab starts: its default plan must match.
    const BwdPlan bp = wkv_backward_plan(1, B, T, C, 0, 0);
    if (bp.nw * bp.L != kCkptSlab) return hipErrorInvalidValue;
    WkvCkptArgs X;
    static_cast<WkvArgs&>(X) = A;
    X.ckpt = reinterpret_cast<uint32_t*>(ckpt);
    X.nck = (T + kCkptSlab - 1) / kCkptSlab;
    ScanGeom g{};
    g.B = B;
    g.T = T;
    g.C = C;
    g.ngrp = (C + 63) / 64;
    g.nslab = (T + kCkptNW * kCkptL - 1) / (kCkptNW * kCkptL);
    g.tag = tag;
    g.spin = spin;
    if (g.nslab > 1) {
        const int64_t nwg = B * g.ngrp * g.nslab;
        const size_t rec = align256((size_t)(nwg * 64) * sizeof(RecordOf<Fwd>::type));
        g.flags = reinterpret_cast<uint64_t*>(ws);
        g.rec_agg = (char*)ws + align256((size_t)nwg * 8);
        g.rec_incl = (char*)g.rec_agg + rec;
    }
    const bool state = A.s_in || A.s_out;
    if (A.r && state) return scan_kernel::launch<WkvCkptOpT<true, true>, 1, kCkptNW, kCkptL>(X, g, sep, st);
    if (A.r) return scan_kernel::launch<WkvCkptOpT<true, false>, 1, kCkptNW, kCkptL>(X, g, sep, st);
    if (state) return scan_kernel::launch<WkvCkptOpT<false, true>, 1, kCkptNW, kCkptL>(X, g, sep, st);
    return scan_kernel::launch<WkvCkptOpT<false, false>, 1, kCkptNW, kCkptL>(X, g, sep, st);
}

}  // namespace linrec

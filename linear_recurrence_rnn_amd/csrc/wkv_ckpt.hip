// wkv_ckpt.hip -- the checkpointing WKV-4 forward on gfx950: y of eq. (14) (RWKV-LLM page,
// "Time-mixing block"), and on the way the forward sums (A, B, A', B') at the end of every
// slab of the backward's gradient kernel, so that a training step's backward can skip its
// own forward pass over k and v (the state kernel).
//
// It is the chunked look-back scan of the plain forward with a wider aggregate: the chunk
// reduction also forms A' and B' (each weight times its distance to the chunk end), slabs
// combine with the float64 fold of wkv_sums.hpp, and the slabs are the gradient kernel's
// (7 chunks of 8 steps).  The look-back's inclusive prefix of slab s is exactly the sums at
// the end of slab s, which the gradient kernel reads at the start of slab s + 1: the
// caller's checkpoint buffer serves as the look-back's inclusive-record array, so keeping the
// sums costs no traffic beyond the records the scan writes anyway.  The re-run of each chunk
// is the plain forward's (A and B rounded to float32 at the chunk's carry-in).
#include "scan_kernel.hpp"
#include "wkv_backward.hpp"
#include "wkv_sums.hpp"

namespace linrec {

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WkvCkptOp {
    using Args = WkvArgs;
    using Base = WkvOp;
    static constexpr bool kReverse = false;
    static constexpr bool kParts = false;
    using Part = NoPart;
    using Chan = Base::Chan;
    using In = Base::In;
    using Local = Base::Local;
    using Agg = Fwd;
    static constexpr int kFloats = 1;
    using Res = Base::Res;

    template <int L>
    __device__ __forceinline__ static Chan chan(const Args& A, int64_t c) { return Base::template chan<L>(A, c); }
    __device__ __forceinline__ static Agg identity() { return fwd_identity(); }
    // No carried state: the sequence starts from the empty sums, and the final state is
    // not written.
    __device__ __forceinline__ static Agg init(const Args&, const ScanGeom&, int64_t, int64_t) {
        return fwd_identity();
    }
    __device__ __forceinline__ static void finish(const Args&, const ScanGeom&, int64_t, int64_t, const Agg&) {}
    __device__ __forceinline__ static Res res(const Args& A, const ScanGeom& g, int64_t b, int64_t row, int64_t col0) {
        return Base::res(A, g, b, row, col0);
    }
    template <int VEC>
    __device__ __forceinline__ static void load(const Res& R, unsigned voff, const Rows& rows, int j, In (&in)[VEC]) {
        Base::template load<VEC>(R, voff, rows, j, in);
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
        Base::Agg c[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) c[e] = {(float)cin[e].a, (float)cin[e].b, cin[e].p};
        return Base::template run<L, VEC>(R, ch, c, in, loc, n, voff, rows);
    }
};

}  // namespace

size_t wkv_ckpt_bytes(int64_t B, int64_t T, int64_t C) {
    const BwdPlan p = wkv_backward_plan(1, B, T, C, 0, 0);
    return (size_t)(B * ((C + 63) / 64) * p.nslab * 64) * sizeof(Fwd);
}

size_t wkv_ckpt_forward_ws_bytes(int64_t B, int64_t T, int64_t C) {
    const BwdPlan p = wkv_backward_plan(1, B, T, C, 0, 0);
    if (p.nslab <= 1) return 0;
    const int64_t nwg = B * ((C + 63) / 64) * p.nslab;
    return align256((size_t)nwg * 8) + align256((size_t)(nwg * 64) * sizeof(Fwd));
}

hipError_t run_wkv_forward_ckpt(const WkvArgs& A, int64_t B, int64_t T, int64_t C, void* ckpt, void* ws,
                                uint64_t tag, int spin, bool sep, hipStream_t st) {
    const BwdPlan p = wkv_backward_plan(1, B, T, C, 0, 0);
    if (p.nw != 7 || p.L != 8) return hipErrorInvalidValue;
    ScanGeom g{};
    g.B = B;
    g.T = T;
    g.C = C;
    g.ngrp = (C + 63) / 64;
    g.nslab = p.nslab;
    g.tag = tag;
    g.spin = spin;
    if (p.nslab > 1) {
        const int64_t nwg = B * g.ngrp * g.nslab;
        g.flags = reinterpret_cast<uint64_t*>(ws);
        g.rec_agg = (char*)ws + align256((size_t)nwg * 8);
        g.rec_incl = ckpt;  // the inclusive prefixes are the checkpoints
    }
    return scan_kernel::launch<WkvCkptOp, 1, 7, 8>(A, g, sep, st);
}

}  // namespace linrec

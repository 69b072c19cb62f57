// wkv_sums.hpp -- the forward sums of WKV-4 that its backward needs, and how they compose.
//
// RWKV-LLM page, "Time-mixing block", eq. (14): with eps = e^{-w} and alpha_i = e^{k_i}, the
// past sums before step t are A_t = sum_{i<t} eps^{t-1-i} alpha_i v_i and B_t (without v).
// The chain rule for w also needs A'_t = sum_{i<t} (t-1-i) eps^{t-1-i} alpha_i v_i and B'_t
// (the pages give no backward; these follow from differentiating A_t and B_t in w).  All four
// share one integer base-2 exponent p (wkv_math.hpp), with float64 mantissas so that long
// folds do not accumulate float32 rounding.
//
// The gradient kernel starts each slab from these sums at the slab's start.  They are found
// either by the backward's own state kernel or, in a training step, by the forward pass that
// keeps them (the checkpointing forward), and both write them in the same record layout: as
// float32 mantissas with the exponent (FwdRec), 20 bytes instead of 36.  The gradient kernel
// scales the slab's starting sums by an exact power of two into float32 for its chunk frame
// anyway, so its fast path sees the same values; its exact path starts from these.
#pragma once

#include "device_common.hpp"
#include "lookback.hpp"
#include "wkv_math.hpp"

namespace linrec {

// Forward sums over a span: A = a 2^p, B = b 2^p, A' = ad 2^p, B' = bd 2^p.
struct Fwd { double a, b, ad, bd; float p; };

__device__ __forceinline__ Fwd fwd_identity() { return {0.0, 0.0, 0.0, 0.0, kEmpty}; }

// The sums kept at a slab boundary (see above).
struct FwdRec { float a, b, ad, bd, p; };

__device__ __forceinline__ FwdRec fwd_to_rec(const Fwd& s) {
    return {(float)s.a, (float)s.b, (float)s.ad, (float)s.bd, s.p};
}
__device__ __forceinline__ Fwd fwd_from_rec(const FwdRec& r) { return {r.a, r.b, r.ad, r.bd, r.p}; }

// Look-back records of these sums (the checkpointing forward's slabs, the state kernel's
// coarse chain) take the same form; the folds stay in float64.
template <>
struct RecordOf<Fwd> {
    using type = FwdRec;
    __device__ __forceinline__ static FwdRec to(const Fwd& s) { return fwd_to_rec(s); }
    __device__ __forceinline__ static Fwd from(const FwdRec& r) { return fwd_from_rec(r); }
};

// State s1, then a span s2 of n2 steps:
//   A = eps^n2 A1 + A2,   A' = eps^n2 (A'1 + n2 A1) + A'2   (B, B' likewise).
__device__ __forceinline__ Fwd fwd_combine(float om, const Fwd& s1, const Fwd& s2, int64_t n2) {
    float p, f1, f2;
    merge_scales(s1.p, (float)s1.b, s2.p, (float)s2.b, mul_split((float)n2, om), p, f1, f2);
    const double g1 = f1, g2 = f2, fn = (double)n2;
    return {fma(s1.a, g1, s2.a * g2), fma(s1.b, g1, s2.b * g2), fma(fma(fn, s1.a, s1.ad), g1, s2.ad * g2),
            fma(fma(fn, s1.b, s1.bd), g1, s2.bd * g2), p};
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

}  // namespace linrec

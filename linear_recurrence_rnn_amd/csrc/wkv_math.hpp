// wkv_math.hpp -- exponent bookkeeping of the WKV-4 sums in float32.
//
// The sums of eq. (14) on the RWKV-LLM page ("Time-mixing block") range over e^{k}, which
// overflows float32 for k > 88.  Every sum is therefore kept as mantissa * 2^p with p an
// INTEGER-valued float (the running maximum exponent rounded up), in base 2:
// kk = k log2(e), om = w log2(e), mu = u log2(e).
//  - Differences of two such exponents are exact, so scale factors 2^{p1-p2} carry no
//    rounding error however large |p| grows (a spike of k = 150 gives p ~ 216, where one
//    float32 ulp is 1.5e-5: re-rounding p at every decay step would cost ~1e-4).
//  - The decay over n steps, n*om, is split into hi + lo (the product and its rounding
//    error), so 2^{(p1 - p) - n om} is accurate to ~1 ulp whenever it is not negligible.
#pragma once

#include "device_common.hpp"

namespace linrec {

// Largest decay rate handled as such; any larger w already makes e^{-w} underflow, and
// the cap keeps n*om finite for every n < 2^31.
constexpr float kMaxOm = 1.0e20f;

struct Split { float hi, lo; };

// n * om = hi + lo exactly (n a small integer-valued float).
__device__ __forceinline__ Split mul_split(float n, float om) {
    const float hi = n * om;
    return {hi, fmaf(n, om, -hi)};
}

// Upper bound, within a factor of 2, of log2(b 2^p) for b >= 0 (b < 2^frexp_exp(b)).
// New integer exponents are chosen from this magnitude rather than from p alone, so a
// decaying state keeps its mantissa in (1/4, 2] instead of drifting towards underflow.
__device__ __forceinline__ float mag(float p, float b) {
    return p + (float)__builtin_amdgcn_frexp_expf(b);
}

// Merge two integer-exponent states: s1 = (b1-weighted, exponent p1) decayed by d = n*om,
// and s2 = (b2, p2), at p = ceil(max(mag1 - d, mag2)).  Returns the scale factors
// f1 = 2^{p1 - d - p} and f2 = 2^{p2 - p}.  b1, b2 >= 0 are the states' positive weight
// sums.  Empty states have p = kEmpty and get a zero factor.
__device__ __forceinline__ void merge_scales(float p1, float b1, float p2, float b2, Split d, float& p,
                                             float& f1, float& f2) {
    p = ceilf(fmaxf(mag(p1, b1) - d.hi, mag(p2, b2)));
    f1 = fast_exp2(((p1 - p) - d.hi) - d.lo);
    f2 = fast_exp2(p2 - p);
}

// A state handed across calls is (a, b, p) with A = a e^p, B = b e^p (natural log, so a
// caller can read it as the past sums of eq. (14)).  Conversions to and from the integer
// base-2 exponent use ln 2 split in two parts, so the exponent's own rounding does not
// scale the state.  a = b = 0 is the empty state.
constexpr float kLn2Hi = 0.693145751953125f, kLn2Lo = 1.42860682030941723212e-6f;

struct Base2State { float a, b, p; };

__device__ __forceinline__ Base2State state_from_natural(float sa, float sb, float sp) {
    if (sa == 0.f && sb == 0.f) return {0.f, 0.f, kEmpty};
    const float P = ceilf(sp * kLog2e);
    const float rem = fmaf(-P, kLn2Lo, fmaf(-P, kLn2Hi, sp));  // sp - P ln 2, in [-ln 2, 0] about
    const float sc = fast_exp2(rem * kLog2e);
    return {sa * sc, sb * sc, P};
}

// The state A = a 2^p as (a', b', p') with p' = float(p ln 2), the rounding of p' compensated
// in a' and b'.
__device__ __forceinline__ void state_to_natural(const Base2State& s, float& oa, float& ob, float& op) {
    if (s.b == 0.f) {
        oa = 0.f;
        ob = 0.f;
        op = 0.f;
        return;
    }
    const float pn = s.p * kLn2Hi + s.p * kLn2Lo;
    const float delta = fmaf(s.p, kLn2Lo, fmaf(s.p, kLn2Hi, -pn));  // p ln 2 - pn
    const float sc = fast_exp2(delta * kLog2e);
    oa = s.a * sc;
    ob = s.b * sc;
    op = pn;
}

}  // namespace linrec

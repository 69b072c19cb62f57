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
// HBM traffic: k, v twice, g once, dL/dk, dL/dv once (28 bytes per element; 20 algorithmic),
// plus the slab-end sums and the reverse look-back records (about 2.5 more at 56-step slabs).
//
// The sums are float64 mantissas times 2^p with p an integer exponent (wkv_math.hpp).  The
// gradients are differences of long sums (v G - H, A' - y B'): float64 mantissas keep their
// rounding from accumulating along the sequence; exponentials, reciprocals and the per-step
// values held in registers stay float32.  On this GPU a float64 FMA issues at the rate of an
// unpacked float32 FMA.
// Every sum over slabs is a fold in chain order (look-back), and dL/dw, dL/du are summed over
// the batch in ascending row order: the results do not depend on scheduling.
#include <atomic>
#include <cstdlib>

#include "chunk_scan.hpp"
#include "device_common.hpp"
#include "lookback.hpp"
#include "wkv_backward.hpp"
#include "wkv_math.hpp"
#include "wkv_sums.hpp"

namespace linrec {

namespace {

__device__ __forceinline__ float gate_sigmoid(float r) { return __builtin_amdgcn_rcpf(1.f + fast_exp2(-r * kLog2e)); }

// Reverse sums: G-like = x 2^r, H-like = h 2^r; z 2^r is the sum of the (positive) weights,
// which x and h can cancel below, and sets the exponent.  z only picks exponents, so float32
// is enough for it (a record is 24 bytes instead of 32).
struct Rev { double x, h; float z, r; };
// Reverse look-back record: the reverse sums of a run of slabs and their dL/dw, dL/du sums.
struct RevRec { Rev st; double sw, su; };

__device__ __forceinline__ Rev rev_identity() { return {0.0, 0.0, 0.f, kEmpty}; }

// Reverse sums: s1 is the state at the end of an earlier span s2 of n2 steps; the result is
// the state at the start of s2:  X = s2 + eps^n2 s1.
__device__ __forceinline__ Rev rev_combine(float om, const Rev& s1, const Rev& s2, int64_t n2) {
    float r, f1, f2;
    merge_scales(s1.r, s1.z, s2.r, s2.z, mul_split((float)n2, om), r, f1, f2);
    const double g1 = f1, g2 = f2;
    return {fma(s1.x, g1, s2.x * g2), fma(s1.h, g1, s2.h * g2), fmaf(s1.z, f1, s2.z * f2), r};
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
    const float p = ceilf(mx);
    // Sums of at most L terms in float32; the carries they feed are float64.
    float a = 0.f, b = 0.f, ad = 0.f, bd = 0.f;
#pragma unroll
    for (int j = 0; j < L; ++j) {
        const float f = fast_exp2(m[j] - p);  // 0 for the unused slots
        const float fd = f * (float)max(n - 1 - j, 0);
        a = fmaf(f, vv[j][e], a);
        b += f;
        ad = fmaf(fd, vv[j][e], ad);
        bd += fd;
    }
    return {a, b, ad, bd, p};
}

// As fwd_chunk, for one channel per lane, keeping the weights: g_j = 2^{m_j - p} replaces
// kk_j, and m0 = m_0 - p (log2 of the first weight).
template <int L>
__device__ __forceinline__ Fwd fwd_chunk_keep(float om, float (&kk)[L], const float (&vv)[L], int n, float& m0) {
    m0 = kEmpty;
    if (n <= 0) return fwd_identity();
    float m[L];
    float mx = kEmpty;
#pragma unroll
    for (int j = 0; j < L; ++j) {
        m[j] = (j < n) ? fmaf(-(float)(n - 1 - j), om, kk[j]) : kEmpty;
        mx = fmaxf(mx, m[j]);
    }
    const float p = ceilf(mx);
    m0 = m[0] - p;
    float a = 0.f, b = 0.f, ad = 0.f, bd = 0.f;
#pragma unroll
    for (int j = 0; j < L; ++j) {
        const float gj = fast_exp2(m[j] - p);  // 0 for the unused slots
        kk[j] = gj;
        const float fd = gj * (float)max(n - 1 - j, 0);
        a = fmaf(gj, vv[j], a);
        b += gj;
        ad = fmaf(fd, vv[j], ad);
        bd += fd;
    }
    return {a, b, ad, bd, p};
}

// Frame of one chunk for the gradient kernel's fast path.  With the chunk's weights
// g_j = 2^{m_j - p} and an INTEGER frame exponent F0, the sums are carried as
//   A~_j = A_{t0+j} 2^{j om - F0}   (B~, A'~, B'~ likewise),
// which decay with the recurrence, so that
//   A~_{j+1} = A~_j + us g_j v_j,  B~_{j+1} = B~_j + us g_j,  A'~_{j+1} = A'~_j + A~_j,
//   the bonus term of step j is cur_j = cs g_j,  D~_j = B~_j + cur_j,
// with us = 2^{p + n om - F0} and cs = 2^{mu + p + (n-1) om - F0}.  In the same frame the
// reverse sums lose their decay too: c_t eps^{t-t0} = (g_t / D~_j) 2^{-F0}, and
//   alpha_s G_s = g_j us (sum_{j' > j} g_{j'} / D~_{j'} + X),   X = G_end 2^{F0 - n om} (carry),
// so the reverse takes no exponential at all.  F0 >= p0 + frexp_exp(b0) and
// >= p + lift + (n-1) om keep every term <= ~1; the carry scale 2^{p0 - F0} is exact.
struct ChunkFrame { float F0, cf, cs, us; bool fast; };

constexpr float kBwdFastLo = -60.f;  // smallest log2 of D~ the fast path accepts
constexpr float kBwdGradMax = 0x1p60f;  // largest |dL/dy| the fast path accepts

__device__ __forceinline__ ChunkFrame chunk_frame(float om, float mu, float lift, const Fwd& cin, float p, float m0,
                                                  int n, float gmax, bool allow) {
    const Split d1 = mul_split((float)(n - 1), om);
    const Split dn = mul_split((float)n, om);
    const float fe = (float)__builtin_amdgcn_frexp_expf((float)cin.b);
    ChunkFrame f;
    f.F0 = fmaxf(cin.p + fe, ceilf((p + lift) + d1.hi));
    f.cf = fast_exp2(cin.p - f.F0);
    const float ls = ((p - f.F0) + d1.hi) + d1.lo;
    f.cs = fast_exp2(ls + mu);
    f.us = fast_exp2(((p - f.F0) + dn.hi) + dn.lo);
    const float carry_lo = ((cin.p - f.F0) + fe) - 1.f;  // B~_0 >= 2^carry_lo
    const float cur_lo = (m0 + ls) + mu;                  // log2 of cur_0
    f.fast = allow && fmaxf(carry_lo, cur_lo) >= kBwdFastLo && gmax < kBwdGradMax;
    return f;
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
        // Slots past n are skipped, not weighted by 0: their values are not defined.
        if (j < n) {
            const float wgt = fast_exp2(m[j] - s.r);
            const double f = wgt * cg[j][e];
            s.x += f;
            s.h = fma(f, (double)ys[j][e], s.h);
            s.z += wgt;
        }
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
    const float r2 = ceilf(fmaxf(mag(s.r, s.z) - om, -q));
    const float f1f = fast_exp2((s.r - r2) - om);
    const double f1 = f1f;
    const float w2 = fast_exp2(-q - r2);
    const double f2 = w2 * c;
    s.x = fma(s.x, f1, f2);
    s.h = fma(s.h, f1, f2 * y);
    s.z = fmaf(s.z, f1f, w2);
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

// ---- a carried state (chain rule of eq. (14) over a sequence cut in pieces) ----
// The state (a, b, p) means A = a e^p, B = b e^p; its gradients are taken w.r.t. (a, b) with
// p held fixed, so that calls chained through the state chain their gradients too.
// 2^r e^x for an integer-valued r: e^x = 2^P e^{x - P ln 2} with ln 2 split in two parts (as
// for the state's exponent), so a large |x| costs no accuracy; 0 for an empty exponent.
__device__ __forceinline__ double pow2_exp(float r, float x) {
    if (r == kEmpty) return 0.0;
    const float P = ceilf(x * kLog2e);
    const float rem = fmaf(-P, kLn2Lo, fmaf(-P, kLn2Hi, x));
    return ldexp((double)fast_exp2(rem * kLog2e), (int)(r + P));
}

// The forward sums before the first token: s_in in base-2 form (empty without it).
__device__ __forceinline__ Fwd fwd_state_in(const WkvBwdArgs& A, const BwdGeom& g, int64_t b, int64_t c) {
    if (!A.s_in) return fwd_identity();
    const float* s = A.s_in + 3 * (b * g.C + c);
    const Base2State x = state_from_natural(s[0], s[1], s[2]);
    if (x.b == 0.f && x.a == 0.f) return fwd_identity();
    return {(double)x.a, (double)x.b, 0.0, 0.0, x.p};
}

// The reverse sums after the last token: G_{T-1} = dL/dA_T = ga' e^{-p'}, H_{T-1} = -dL/dB_T.
__device__ __forceinline__ Rev rev_state_out(const WkvBwdArgs& A, const BwdGeom& g, int64_t b, int64_t c) {
    if (!A.gs_out) return rev_identity();
    const float ga = A.gs_out[2 * (b * g.C + c)], gb = A.gs_out[2 * (b * g.C + c) + 1];
    if (ga == 0.f && gb == 0.f) return rev_identity();
    // e^{-p'} = 2^P 2^{rem log2 e}, P integer, rem = -p' - P ln 2 with ln 2 split in two parts.
    const float np = -A.s_out[3 * (b * g.C + c) + 2];
    const float P = ceilf(np * kLog2e);
    const float rem = fmaf(-P, kLn2Lo, fmaf(-P, kLn2Hi, np));
    const double sc = (double)fast_exp2(rem * kLog2e);
    return {ga * sc, -(double)gb * sc, (float)((fabs((double)ga) + fabs((double)gb)) * sc), P};
}

// dL/dw's share of the state after the last token: -(dL/dA_T A'_T + dL/dB_T B'_T), with the
// forward sums at the end of the sequence.
__device__ __forceinline__ double sw_state_out(const WkvBwdArgs& A, const BwdGeom& g, int64_t b, int64_t c,
                                               const Fwd& end) {
    if (!A.gs_out) return 0.0;
    const double ga = A.gs_out[2 * (b * g.C + c)], gb = A.gs_out[2 * (b * g.C + c) + 1];
    return -(ga * end.ad + gb * end.bd) * pow2_exp(end.p, -A.s_out[3 * (b * g.C + c) + 2]);
}

// dL/d(a, b) of s_in from the reverse sums before the first token (G_{-1}, H_{-1}).
__device__ __forceinline__ void write_state_grad(const WkvBwdArgs& A, const BwdGeom& g, int64_t b, int64_t c,
                                                 const Rev& st) {
    const double f = pow2_exp(st.r, A.s_in ? A.s_in[3 * (b * g.C + c) + 2] : 0.f);
    A.gs_in[2 * (b * g.C + c)] = (float)(st.x * f);
    A.gs_in[2 * (b * g.C + c) + 1] = (float)(-st.h * f);
}

// Forward sums at the start of slab s: written by the state kernel at the end of slab s-1;
// before the first slab, the carried state (STATE) or the empty one.
template <int VEC, bool STATE>
__device__ __forceinline__ void fwd_carry_in(const WkvBwdArgs& A, const BwdGeom& g, int64_t gi, int64_t b,
                                             int64_t c0, int64_t s, int lane, bool active, Fwd (&x)[VEC]) {
    constexpr int64_t per = 64 * VEC * kDwords<FwdRec>;  // dwords per slab record
    if (s > 0 && active) {
        FwdRec r[VEC];
        load_record<VEC>(reinterpret_cast<const uint32_t*>(g.incl_f) + gi * g.nslab * per, s - 1, lane, r);
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[e] = fwd_from_rec(r[e]);
    } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[e] = (STATE && active) ? fwd_state_in(A, g, b, c0 + e) : fwd_identity();
    }
}

// Steps of chunk x of a slab of slab_n steps (0 for chunks past the end).
template <int L>
__device__ __forceinline__ int chunk_len(int x, int slab_n) {
    return max(0, min(L, slab_n - x * L));
}

// ------------------------------------------------------------------------------------
// State kernel: the forward sums at the end of slabs 0 .. nslab-2 (the gradient kernel's
// slabs, "fine" slabs of SLAB = NW * L steps), for one channel per lane.  Persistent.
//
// An item is kStateFine consecutive fine slabs of one sequence; items form a coarse chain
// with its own decoupled look-back.  Compute wave w streams fine slab w of the item in
// L-step chunks (the loads of the next chunk are issued before the current one is reduced)
// and folds it into the slab's sums; the coordinator folds the slabs into the item's
// aggregate, publishes it, looks back over the earlier items and, from the carry, writes the
// sums at every fine slab end and publishes the item's inclusive prefix.  The grid holds
// only workgroups that are resident together; workgroup i takes items i, i + grid, ... in
// chain-major order, so an item's predecessors come earlier in every workgroup's sequence.
// LDS is double-buffered between the two roles, which meet at one barrier per item.
// ------------------------------------------------------------------------------------
constexpr int kStateFine = 7;

// As fwd_chunk, for one channel per lane (kk = k log2 e).
template <int L>
__device__ __forceinline__ Fwd fwd_chunk1(float om, const float (&kk)[L], const float (&vv)[L], int n) {
    if (n <= 0) return fwd_identity();
    float m[L];
    float mx = kEmpty;
#pragma unroll
    for (int j = 0; j < L; ++j) {
        m[j] = (j < n) ? fmaf(-(float)(n - 1 - j), om, kk[j]) : kEmpty;
        mx = fmaxf(mx, m[j]);
    }
    const float p = ceilf(mx);
    float a = 0.f, b = 0.f, ad = 0.f, bd = 0.f;
#pragma unroll
    for (int j = 0; j < L; ++j) {
        const float f = fast_exp2(m[j] - p);
        const float fd = f * (float)max(n - 1 - j, 0);
        a = fmaf(f, vv[j], a);
        b += f;
        ad = fmaf(fd, vv[j], ad);
        bd += fd;
    }
    return {a, b, ad, bd, p};
}

// 6 waves per SIMD (<= 80 VGPRs, no spills): three workgroups resident per CU.
template <int NW, int L>
__global__ __launch_bounds__(64 * (kStateFine + 1)) __attribute__((amdgpu_waves_per_eu(6)))
void wkv_bwd_state_kernel(WkvBwdArgs A, BwdGeom g) {
    constexpr int SLAB = NW * L;
    constexpr int F = kStateFine;
    constexpr int kRec = 64 * kRecDwords<Fwd>;  // dwords per coarse-chain record
    __shared__ Fwd shf[2][F][64];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int64_t G = g.B * g.ngrp;
    const int64_t nfine = g.nslab - 1;             // fine slabs whose end state is needed
    const int64_t nitem = (nfine + F - 1) / F;     // coarse chain length
    const int64_t items = G * nitem;
    const unsigned rowb = (unsigned)(g.C * 4);
    const unsigned voff = (unsigned)(lane * 4);
    const int64_t total = g.B * g.T * g.C;
    // Item u = q G + b ngrp + grp.  This workgroup's items u_i = blockIdx + i grid are
    // decomposed once and then advanced by the decomposed grid step, so the walk divides
    // nothing (a 64-bit division is a long scalar sequence, and it ran twice per chunk).
    struct Item { int64_t q, gi, b, grp, c0; bool active; };
    const int64_t ugrid = gridDim.x;
    const int64_t dq = ugrid / G, dgi = ugrid - dq * G;
    const int64_t db = dgi / g.ngrp, dgrp = dgi - db * g.ngrp;
    auto settle = [&](Item& it) {
        it.gi = it.b * g.ngrp + it.grp;
        it.c0 = it.grp * 64 + lane;
        it.active = it.c0 < g.C;
    };
    auto first_item = [&]() {
        Item it;
        it.q = (int64_t)blockIdx.x / G;
        const int64_t gi = (int64_t)blockIdx.x - it.q * G;
        it.b = gi / g.ngrp;
        it.grp = gi - it.b * g.ngrp;
        settle(it);
        return it;
    };
    auto next_item = [&](Item it) {  // u -> u + grid
        it.grp += dgrp;
        it.b += db;
        if (it.grp >= g.ngrp) {
            it.grp -= g.ngrp;
            ++it.b;
        }
        it.q += dq;
        if (it.b >= g.B) {
            it.b -= g.B;
            ++it.q;
        }
        settle(it);
        return it;
    };

    if (w < F) {
        // This workgroup's items are u_i = blockIdx + i * grid; the wave walks the chunks of
        // its fine slab in each, t = i * NW + c.
        const int64_t my_items = blockIdx.x < items ? (items - 1 - blockIdx.x) / gridDim.x + 1 : 0;
        const int64_t nt = my_items * NW;
        float kk[2][L], vv[2][L], wr[2];
        Item iss = first_item();  // chunk c_iss of item iss is the next to be issued
        int c_iss = 0;
        auto issue = [&](int bs) {
            const Item it = iss;
            const int c = c_iss;
            if (++c_iss == NW) {
                c_iss = 0;
                iss = next_item(iss);
            }
            const int64_t f = it.q * F + w;
            const bool valid = it.active && f < nfine;
            const int64_t base = (it.b * g.T + f * SLAB + (int64_t)c * L) * g.C + it.grp * 64;
            const rsrc_t rk = make_rsrc(A.k + base, (total - base) * 4), rv = make_rsrc(A.v + base, (total - base) * 4);
            wr[bs] = it.active ? A.w[it.c0] : 0.f;
#pragma unroll
            for (int j = 0; j < L; ++j) {
                kk[bs][j] = valid ? ldb<1>(rk, voff, j * rowb).v[0] : 0.f;
                vv[bs][j] = valid ? ldb<1>(rv, voff, j * rowb).v[0] : 0.f;
            }
        };
        Fwd acc = fwd_identity();
        int ib = 0;
        Item cur = first_item();  // chunk c_cur of item cur is the next to be reduced
        int c_cur = 0;
        auto step = [&](int64_t t, int bs) {
            const Item it = cur;
            const int c = c_cur;
            if (++c_cur == NW) {
                c_cur = 0;
                cur = next_item(cur);
            }
            const bool valid = it.active && it.q * F + w < nfine;
            const float om = fminf(wr[bs] * kLog2e, kMaxOm);
            float kl[L];
#pragma unroll
            for (int j = 0; j < L; ++j) kl[j] = kk[bs][j] * kLog2e;
            const Fwd chunk = fwd_chunk1<L>(om, kl, vv[bs], valid ? L : 0);
            if (t + 1 < nt) issue(bs ^ 1);
            acc = (c == 0) ? chunk : fwd_combine(om, acc, chunk, L);
            if (c == NW - 1) {
                shf[ib][w][lane] = acc;
                __syncthreads();  // the item's fine-slab sums are in shf[ib]
                ib ^= 1;
            }
        };
        if (nt > 0) issue(0);
        for (int64_t t = 0; t < nt; t += 2) {
            step(t, 0);
            if (t + 1 < nt) step(t + 1, 1);
        }
        return;
    }

    // ---- coordinator ----
    int ib = 0;
    Item it = first_item();
    for (int64_t u = blockIdx.x; u < items; u += gridDim.x, ib ^= 1, it = next_item(it)) {
        float om[1], mu[1];
        load_chan<1>(A, it.c0, it.active, om, mu);
        const Chain<Fwd> chn{g.flags_c + it.gi * nitem, reinterpret_cast<uint32_t*>(g.agg_c) + it.gi * nitem * kRec,
                             reinterpret_cast<uint32_t*>(g.incl_c) + it.gi * nitem * kRec, g.tag_f, g.spin};
        const int64_t f0 = it.q * F;
        const int nvalid = (int)((nfine - f0) < F ? (nfine - f0) : F);
        __syncthreads();
        const uint64_t first = prefetch_window(chn, it.q, lane);  // overlaps the fold below
        // Chain values (the item's aggregate, each fold, the inclusive sums) are taken in the
        // records' form, and the inclusive sums are the carry folded with that aggregate, so
        // that every look-back path folds the same values (lookback.hpp).
        Fwd mine[1], carry[1];
        mine[0] = shf[ib][0][lane];
        for (int x = 1; x < nvalid; ++x) mine[0] = fwd_combine(om[0], mine[0], shf[ib][x][lane], SLAB);
        mine[0] = as_record(mine[0]);
        carry[0] = as_record(it.active ? fwd_state_in(A, g, it.b, it.c0) : fwd_identity());
        const bool has_succ = it.q + 1 < nitem;
        if (has_succ) publish<1>(chn, it.q, lane, mine, false);
        auto fold = [&](Fwd (&c)[1], const Fwd (&x)[1], int64_t) {
            c[0] = as_record(fwd_combine(om[0], c[0], x[0], (int64_t)F * SLAB));  // earlier items are full
        };
        auto recompute = [&](int64_t jj, Fwd (&x)[1]) {
            const int64_t bj = (it.b * g.T + jj * F * SLAB) * g.C + it.grp * 64;
            const rsrc_t rkj = make_rsrc(A.k + bj, (total - bj) * 4), rvj = make_rsrc(A.v + bj, (total - bj) * 4);
            x[0] = fwd_identity();
            if (it.active) {
                for (int t = 0; t < F * SLAB; ++t) {
                    const float kj = ldb<1>(rkj, voff, t * rowb).v[0] * kLog2e;
                    const float vj = ldb<1>(rvj, voff, t * rowb).v[0];
                    fwd_advance(om[0], x[0], kj, (double)vj, mag(x[0].p, (float)x[0].b));
                }
            }
            x[0] = as_record(x[0]);  // as if read
        };
        look_back<1, 2>(chn, it.q, lane, carry, fold, recompute, first);
        if (has_succ) {
            const Fwd incl[1] = {as_record(fwd_combine(om[0], carry[0], mine[0], (int64_t)F * SLAB))};
            publish<1>(chn, it.q, lane, incl, true);
        }
        // The sums at the end of every fine slab of the item (read by the gradient kernel).
        uint32_t* fine = reinterpret_cast<uint32_t*>(g.incl_f) + it.gi * g.nslab * (64 * kDwords<FwdRec>);
        for (int x = 0; x < nvalid; ++x) {
            carry[0] = fwd_combine(om[0], carry[0], shf[ib][x][lane], SLAB);
            const FwdRec r[1] = {fwd_to_rec(carry[0])};
            store_record<1>(fine, f0 + x, lane, r);
        }
    }
}

// The reverse record of chain slab jj computed from its inputs (the look-back's fallback
// when the slab has not published in time): the slab's forward re-run from the state
// kernel's sums, one step at a time, accumulating its reverse sums in time order.
template <int VEC, int SLAB, bool STATE>
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
    const rsrc_t rrj = make_rsrc(A.r ? A.r + bj : A.gy + bj, A.r ? (total - bj) * 4 : 0);
    Fwd fs[VEC];
    const int64_t c0 = grp * CW + (int64_t)lane * VEC;
    fwd_carry_in<VEC, STATE>(A, g, gi, b, c0, sj, lane, active, fs);
#pragma unroll
    for (int e = 0; e < VEC; ++e) x[e] = {rev_identity(), 0.0, 0.0};
    if (!active) return;
    for (int t = 0; t < nj; ++t) {
        const FV<VEC> kt = ldb<VEC>(rkj, voff, t * rowb), vt = ldb<VEC>(rvj, voff, t * rowb);
        FV<VEC> gt = ldb<VEC>(rgj, voff, t * rowb);
        if (A.r) {
            const FV<VEC> rt = ldb<VEC>(rrj, voff, t * rowb);
#pragma unroll
            for (int e = 0; e < VEC; ++e) gt.v[e] *= gate_sigmoid(rt.v[e]);
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const StepOut o = fwd_step(om[e], mu[e], fs[e], kt.v[e] * kLog2e, vt.v[e], gt.v[e], x[e].sw, x[e].su);
            const Rev one{(double)o.c, (double)o.c * (double)o.y, 1.f, -o.q};
            x[e].st = rev_combine(om[e], one, x[e].st, t);
        }
    }
    if (STATE && jj == 0) {
        // The last slab of the sequence: its record also holds the final state's gradient
        // (the reverse sums behind the slab and dL/dw's share).
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            x[e].st = rev_combine(om[e], rev_state_out(A, g, b, c0 + e), x[e].st, nj);
            x[e].sw += sw_state_out(A, g, b, c0 + e, fs[e]);
        }
    }
}

// ------------------------------------------------------------------------------------
// Gradient kernel: slabs in reverse time order (chain position q = nslab-1-s).  Waves
// 0 .. NW-1 own one chunk each and hold its inputs and per-step values in registers; wave
// NW (the coordinator) handles the slab's records:
//   B1  chunks' forward sums in shf,     -> each chunk folds its own carry-in from them; the
//       the slab's start in sh_cin          coordinator tries the reverse look-back meanwhile
//   B3  chunks' reverse sums in shr, and -> coordinator: the reverse sums at the slab's end
//       their dL/dw, dL/du in shwu           in sh_rend -- at once when the early look-back
//                                           found the carry, the slab's records being formed
//                                           and published after B4 while the chunks run;
//                                           otherwise after publishing the aggregate and the
//                                           look-back
//   B4                                   -> each chunk folds the reverse sums at its own end
// The two roles are separate branches, so the look-back's registers do not add to those
// of the chunk data.
// ------------------------------------------------------------------------------------
// Register budget: with 8-step chunks the kernel fits 80 VGPRs (6 waves per SIMD), so three
// 8-wave workgroups share a CU; that hides one workgroup's look-back behind the others'
// work better than the compiler's own choice (~90 VGPRs, two workgroups).
template <int L, bool GATE, bool STATE>
constexpr int grad_waves_per_eu() {
    // Every instance fits: the gate's r_j live only until the fast path has written dL/dr
    // (the exact path reads r again), and the state's terms are formed where few chunk
    // values are live.
    return L <= 8 ? 6 : 1;
}

// GATE: the output is sigma(r) wkv (eq. (15)); dL/dwkv = gy sigma(r) drives every sum, and
// dL/dr = dL/dwkv wkv sigma(-r) is written where wkv is formed.  STATE: a carried state
// s_in starts the forward sums, the final state's gradient gs_out starts the reverse ones and
// gs_in is written.  Separate instances, so the plain kernel's registers are unchanged.
// G3: the grid is (ngrp, B, nslab); otherwise flat (sizes beyond the 3-D grid's limits).
template <int VEC, int NW, int L, bool GATE, bool STATE, bool G3>
__global__ __launch_bounds__(64 * (NW + 1))
__attribute__((amdgpu_waves_per_eu(grad_waves_per_eu<L, GATE, STATE>())))
void wkv_bwd_grad_kernel(WkvBwdArgs A, BwdGeom g) {
    constexpr int CW = 64 * VEC;
    constexpr int SLAB = NW * L;
    __shared__ Fwd shf[NW][CW];
    __shared__ Rev shr[NW][CW];
    __shared__ double shwu[NW][CW][2];
    __shared__ RevRec sh_mine[CW];
    __shared__ int sh_done;  // compute waves past their forward re-run (the coordinator's cue)
    __shared__ RevRec sh_carry[CW];  // the reverse carry, when found before B3
    __shared__ Fwd sh_cin[CW];       // the forward sums at the slab's start
    __shared__ Rev sh_rend[CW];      // the reverse sums at the slab's end

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    // Chain position q (later slabs first), batch row b and channel group grp: from a 3-D
    // grid (ngrp, B, nslab) directly, or by dividing the flat grid's block index, a long
    // scalar sequence ahead of the first load.
    int64_t q, b, grp;
    if constexpr (G3) {
        q = blockIdx.z;
        b = blockIdx.y;
        grp = blockIdx.x;
    } else {
        const int64_t G = g.B * g.ngrp;
        q = (int64_t)blockIdx.x / G;
        const int64_t gq = (int64_t)blockIdx.x - q * G;
        b = gq / g.ngrp;
        grp = gq - b * g.ngrp;
    }
    const int64_t gi = b * g.ngrp + grp;
    const int64_t s = g.nslab - 1 - q;
    const int64_t c0 = grp * CW + (int64_t)lane * VEC;
    const bool active = c0 < g.C;
    const int64_t t_slab = s * SLAB;
    const int slab_n = (int)((g.T - t_slab) < SLAB ? (g.T - t_slab) : SLAB);

    float om[VEC], mu[VEC];
    load_chan<VEC>(A, c0, active, om, mu);

    if (w < NW) {
        static_assert(VEC == 1, "the gradient kernel keeps one channel per lane");
        const int n = active ? chunk_len<L>(w, slab_n) : 0;
        const unsigned rowb = (unsigned)(g.C * 4);
        const unsigned voff = (unsigned)(lane * 4);
        const int64_t total = g.B * g.T * g.C;
        const int64_t base = (b * g.T + t_slab + (int64_t)w * L) * g.C + grp * CW;
        const int64_t nbytes = (total - base) * 4;
        const rsrc_t rk = make_rsrc(A.k + base, nbytes), rg = make_rsrc(A.gy + base, nbytes);
        // Per step: sa = g_j (fast path) or q_j (exact path); vv = v_j; sc = dL/dy_j, then
        // g_j / D~_j (fast) or g_j / dm_j (exact); sy = y_j; sd = v_j - y_j.
        float sa[L], vv[L], sc[L], sy[L], sd[L];
        float rr[GATE ? L : 1];  // r_j
        const rsrc_t rgr = make_rsrc(GATE ? A.gr + base : A.gk + base, GATE ? nbytes : 0);
        const rsrc_t rrs = make_rsrc(GATE ? A.r + base : A.k + base, GATE ? nbytes : 0);
        float gmax = 0.f;
        {
            const rsrc_t rv = make_rsrc(A.v + base, nbytes);
#pragma unroll
            for (int j = 0; j < L; ++j) {
                float kt = 0.f, vt = 0.f, gt = 0.f;
                if (j < n) {
                    kt = ldb<1>(rk, voff, j * rowb).v[0];
                    vt = ldb<1>(rv, voff, j * rowb).v[0];
                    gt = ldb<1>(rg, voff, j * rowb).v[0];
                }
                if constexpr (GATE) {
                    rr[j] = j < n ? ldb<1>(rrs, voff, j * rowb).v[0] : 0.f;
                    gt *= gate_sigmoid(rr[j]);
                }
                sa[j] = kt * kLog2e;
                vv[j] = vt;
                sc[j] = gt;
                gmax = fmaxf(gmax, fabsf(gt));
            }
        }
        float m0;
        shf[w][lane] = fwd_chunk_keep<L>(om[0], sa, vv, n, m0);
        const float p_chunk = shf[w][lane].p;
        __syncthreads();  // B1: every chunk's sums are in shf, the slab's start in sh_cin
        // My chunk's carry-in: the slab's start followed by the chunks before mine, folded by
        // this wave itself (the waves' folds run side by side, none waits for another).
        Fwd cin = sh_cin[lane];
        for (int x = 0; x < w; ++x) cin = fwd_combine(om[0], cin, shf[x][lane], chunk_len<L>(x, slab_n));
        if constexpr (STATE) {
            // The last slab: dL/dw's share of the final state takes the sums at the slab's
            // end, which the last wave extends its own carry-in to (the same fold as the
            // other waves').  The coordinator adds it to the slab's record after B3.
            if (q == 0 && w == NW - 1) {
                sh_mine[lane].sw =
                    active ? sw_state_out(A, g, b, c0, fwd_combine(om[0], cin, shf[w][lane], chunk_len<L>(w, slab_n)))
                           : 0.0;
            }
        }

        const float lift = ceilf(fmaxf(fmaxf(om[0], mu[0]), 0.f));
        ChunkFrame fr = chunk_frame(om[0], mu[0], lift, cin, p_chunk, m0, n, gmax, n > 0 && !g.exact_only);
        double sw = 0.0, su = 0.0;
        Rev ragg = rev_identity();
        if (fr.fast) {
            // Forward in the frame (float32: at most L terms are added to the converted
            // carry).  Also the chunk's reverse sums seen from its start:
            // x = sum g/D~, h = sum g y/D~, z = sum 1/D~, at exponent -F0.
            const double cf = fr.cf;
            float a = (float)(cin.a * cf), bb = (float)(cin.b * cf), ad = (float)(cin.ad * cf),
                  bd = (float)(cin.bd * cf);
            float x = 0.f, h = 0.f, z = 0.f, swf = 0.f, suf = 0.f, dmin = 1.f;
#pragma unroll
            for (int j = 0; j < L; ++j) {
                if (j < n) {
                    const float gj = sa[j], vj = vv[j];
                    const float cur = gj * fr.cs;
                    const float dt = bb + cur;
                    const float inv = __builtin_amdgcn_rcpf(dt);
                    dmin = fminf(dmin, dt);
                    const float y = fmaf(cur, vj, a) * inv;
                    const float vmy = fmaf(vj, bb, -a) * inv;
                    if constexpr (GATE) {
                        FV<1> o;
                        o.v[0] = sc[j] * y * gate_sigmoid(-rr[j]);
                        stb<1>(rgr, voff, j * rowb, o);
                    }
                    const float cg = sc[j] * inv;
                    swf = fmaf(-cg, fmaf(-y, bd, ad), swf);
                    suf = fmaf(cg * cur, vmy, suf);
                    x += cg;
                    h = fmaf(cg, y, h);
                    z += inv;
                    const float up = gj * fr.us;
                    ad += a;
                    bd += bb;
                    a = fmaf(up, vj, a);
                    bb += up;
                    sc[j] = cg;
                    sy[j] = y;
                    sd[j] = vmy;
                }
            }
            ragg = {x, h, z, -fr.F0};
            sw = swf;
            su = suf;
            // A denominator below 2^kBwdFastLo would let g / D~ leave float range: redo exactly.
            fr.fast = dmin >= 0x1p-60f;
            if (!fr.fast) {
                sw = 0.0;
                su = 0.0;
            }
        }
        if (!fr.fast && n > 0) {
            // Exact per-step path (wkv_math.hpp exponents); k, dL/dy and r are read again, so
            // that no register holds r past the fast path.
            Fwd st = cin;
#pragma unroll
            for (int j = 0; j < L; ++j) {
                if (j < n) {
                    const float kj = ldb<1>(rk, voff, j * rowb).v[0] * kLog2e;
                    float gj = ldb<1>(rg, voff, j * rowb).v[0];
                    const float rj = GATE ? ldb<1>(rrs, voff, j * rowb).v[0] : 0.f;
                    if constexpr (GATE) gj *= gate_sigmoid(rj);
                    const StepOut o = fwd_step(om[0], mu[0], st, kj, vv[j], gj, sw, su);
                    if constexpr (GATE) {
                        // Overwrites the fast path's value when that path was abandoned.
                        FV<1> og;
                        og.v[0] = gj * o.y * gate_sigmoid(-rj);
                        stb<1>(rgr, voff, j * rowb, og);
                    }
                    sa[j] = o.q;
                    sc[j] = o.c;
                    sy[j] = o.y;
                    sd[j] = o.vmy;
                }
            }
            float qs[L][1], cg[L][1], ys[L][1];
#pragma unroll
            for (int j = 0; j < L; ++j) {
                qs[j][0] = sa[j];
                cg[j][0] = sc[j];
                ys[j][0] = sy[j];
            }
            ragg = rev_chunk<L, 1>(om[0], qs, cg, ys, 0, n);
        }
        shwu[w][lane][0] = sw;
        shwu[w][lane][1] = su;
        shr[w][lane] = ragg;
        if (lane == 0) __hip_atomic_fetch_add(&sh_done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __syncthreads();  // B3
        if (fr.fast && n > 0) {
            // The chunk's own part of the reverse re-run, while the coordinator looks back
            // for the carry: with S_s the frame sums after step s in the chunk,
            //   dL/dv_s = (g beta / D)_s + g_s us S^x_s + [g_s X],
            //   dL/dk_s = (g beta / D)_s (v - y)_s + g_s us (v_s S^x_s - S^h_s) + [g_s (v_s X - H)],
            // the bracketed carry terms are added after B4.  sy and sd take the partial sums.
            float Sx = 0.f, Sh = 0.f;
#pragma unroll
            for (int j = L - 1; j >= 0; --j) {
                if (j < n) {
                    const float gj = sa[j], vj = vv[j];
                    const float gus = gj * fr.us;
                    const float cc = sc[j] * (gj * fr.cs);  // g beta / D
                    const float gvl = fmaf(gus, Sx, cc);
                    const float gkl = fmaf(cc, sd[j], gus * fmaf(vj, Sx, -Sh));
                    Sx += sc[j];
                    Sh = fmaf(sc[j], sy[j], Sh);
                    sy[j] = gvl;
                    sd[j] = gkl;
                }
            }
        }
        __syncthreads();  // B4: the reverse sums at the slab's end are in sh_rend

        // Reverse re-run of my chunk; the outputs replace v and dL/dy's slot.
        if (n > 0) {
            // The reverse sums at my chunk's end: the slab's end followed (backwards) by the
            // chunks after mine, folded by this wave itself.
            Rev rc = sh_rend[lane];
            for (int x = NW - 1; x > w; --x) rc = rev_combine(om[0], rc, shr[x][lane], chunk_len<L>(x, slab_n));
            if (fr.fast) {
                // Carry in frame units, X = x_c 2^{r_c + F0 - n om}, pre-multiplied by us:
                // alpha_s G_s = g_s (us X + us S_s) with S_s the frame sum after s in the chunk.
                // The carry part of v X - H cancels, so it is formed in float64.
                double Xs = 0.0, Hs = 0.0;
                if (rc.x != 0.0 || rc.h != 0.0) {
                    const Split dn = mul_split((float)n, om[0]);
                    const float e = ((rc.r + fr.F0) - dn.hi) - dn.lo;
                    const float ei = floorf(e);
                    const double kap = ldexp((double)(fast_exp2(e - ei) * fr.us), (int)ei);
                    Xs = rc.x * kap;
                    Hs = rc.h * kap;
                }
                const float Xsf = (float)Xs;
#pragma unroll
                for (int j = L - 1; j >= 0; --j) {
                    if (j < n) {
                        const float gj = sa[j], vj = vv[j];
                        const float tc = (float)fma((double)vj, Xs, -Hs);
                        sa[j] = fmaf(gj, tc, sd[j]);
                        vv[j] = fmaf(gj, Xsf, sy[j]);
                    }
                }
            } else {
                Rev rs = rc;
#pragma unroll
                for (int j = L - 1; j >= 0; --j) {
                    if (j < n) {
                        const float kj = ldb<1>(rk, voff, j * rowb).v[0] * kLog2e;
                        float gk, gv;
                        rev_step(om[0], mu[0], rs, kj, vv[j], sc[j], sa[j], sy[j], sd[j], gk, gv);
                        sa[j] = gk;
                        vv[j] = gv;
                    }
                }
            }
            const rsrc_t rgk = make_rsrc(A.gk + base, nbytes), rgv = make_rsrc(A.gv + base, nbytes);
#pragma unroll
            for (int j = 0; j < L; ++j) {
                if (j < n) {
                    FV<1> ok, ov;
                    ok.v[0] = sa[j];
                    ov.v[0] = vv[j];
                    stb<1>(rgk, voff, j * rowb, ok);
                    stb<1>(rgv, voff, j * rowb, ov);
                }
            }
        }
        return;
    }

    // ---- coordinator ----
    if (lane == 0) sh_done = 0;
    {
        // The slab's start: the previous slab's sums (state kernel), or the carried state.
        Fwd cin[VEC];
        fwd_carry_in<VEC, STATE>(A, g, gi, b, c0, s, lane, active, cin);
#pragma unroll
        for (int e = 0; e < VEC; ++e) sh_cin[lane * VEC + e] = cin[e];
    }
    __syncthreads();  // B1
    const Chain<RevRec> chn{g.flags_r + gi * g.nslab,
                            reinterpret_cast<uint32_t*>(g.agg_r) + gi * g.nslab * (CW * kDwords<RevRec>),
                            reinterpret_cast<uint32_t*>(g.incl_r) + gi * g.nslab * (CW * kDwords<RevRec>), g.tag_r,
                            g.spin};
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
    // While the chunks re-run the forward, look back for the reverse carry: the later slabs
    // have usually published by then, and the carry is then ready when the chunks' sums are.
    bool early;
    {
        RevRec c[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) c[e] = {rev_identity(), 0.0, 0.0};
        early = try_look_back<VEC>(chn, q, lane, c, fold, [&]() {
            return __hip_atomic_load(&sh_done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= NW;
        });
#pragma unroll
        for (int e = 0; e < VEC; ++e) sh_carry[lane * VEC + e] = c[e];  // parked across B3 (registers)
    }
    __syncthreads();  // B3
    // The reverse sums at the slab's end: the carry (the last slab: the final state's
    // gradient, which its record holds as well).
    auto slab_end = [&](const RevRec (&cr)[VEC]) {
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            sh_rend[lane * VEC + e] = (STATE && q == 0 && active) ? rev_state_out(A, g, b, c0 + e) : cr[e].st;
    };
    RevRec mine[VEC], carry[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) carry[e] = sh_carry[lane * VEC + e];  // the carry, or the empty one
    if (early) {
        // The chunks need only the carry: let them run, then form and publish the records.
        slab_end(carry);
        __syncthreads();  // B4
    }
    const uint64_t first = early ? 0 : prefetch_window(chn, q, lane);  // overlaps the slab fold
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        // Reverse sums of the slab from its start: chunks folded from the last to the first.
        Rev a = rev_identity();
        double sw = 0.0, su = 0.0;
        // The last slab's record also holds the final state's gradient, so that every chain
        // starts from the empty carry.
        if (STATE && q == 0 && active) a = sh_rend[lane * VEC + e];  // set by slab_end (q = 0 is early)
        for (int x = NW - 1; x >= 0; --x) a = rev_combine(om[e], a, shr[x][lane * VEC + e], chunk_len<L>(x, slab_n));
        for (int x = 0; x < NW; ++x) {
            sw += shwu[x][lane * VEC + e][0];
            su += shwu[x][lane * VEC + e][1];
        }
        if (STATE && q == 0) sw += sh_mine[lane * VEC + e].sw;  // the final state's share (last wave)
        mine[e] = {a, sw, su};
        sh_mine[lane * VEC + e] = mine[e];  // kept in LDS across the look-back (registers)
    }
    const bool has_succ = s > 0;
    // With the carry already known the inclusive record follows at once: the aggregate would
    // only cost the workgroup one more write round trip before its slot is released.
    if (has_succ && !early) publish<VEC>(chn, q, lane, mine, false);
    if (!early) {
        auto recompute = [&](int64_t jj, RevRec (&x)[VEC]) {
            rev_record_from_inputs<VEC, SLAB, STATE>(A, g, jj, gi, b, grp, lane, active, om, mu, x);
        };
        look_back<VEC, 1>(chn, q, lane, carry, fold, recompute, first);
    }
    RevRec incl[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        incl[e] = carry[e];
        mine[e] = sh_mine[lane * VEC + e];
    }
    fold(incl, mine, q);
    if (has_succ) {
        publish<VEC>(chn, q, lane, incl, true);
    } else if (active) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            g.part[2 * (b * g.C + c0 + e)] = incl[e].sw;
            g.part[2 * (b * g.C + c0 + e) + 1] = incl[e].su;
            if (STATE && A.gs_in) write_state_grad(A, g, b, c0 + e, incl[e].st);  // the sequence's first slab
        }
    }
    if (!early) {
        slab_end(carry);
        __syncthreads();  // B4
    }
}

// gw[c] = sum_b part[b, c].w, gu likewise, in ascending b.  The rows are loaded 8 at a time
// (one 16-byte load per row) and then added in order: one memory round trip per 8 rows
// where a load feeding each add cost one per row (B = 8: 4.7 us).  The same association,
// so the same bits.
__global__ __launch_bounds__(256) void wkv_bwd_wu_kernel(const double* __restrict__ part, int64_t B,
                                                         int64_t C, float* __restrict__ gw,
                                                         float* __restrict__ gu) {
    constexpr int K = 8;
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= C) return;
    const double2* p2 = reinterpret_cast<const double2*>(part);
    double sw = 0.0, su = 0.0;
    for (int64_t b0 = 0; b0 < B; b0 += K) {
        double2 x[K];
#pragma unroll
        for (int i = 0; i < K; ++i) x[i] = (b0 + i < B) ? p2[(b0 + i) * C + c] : double2{0.0, 0.0};
#pragma unroll
        for (int i = 0; i < K; ++i) {
            if (b0 + i < B) {
                sw += x[i].x;
                su += x[i].y;
            }
        }
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

// Workgroups of `kernel` (block of `threads`) that the current device holds at once: blocks
// per CU from the occupancy query times the CU count, cached per device in `cache` (one
// cache per kernel).
constexpr int kMaxDev = 64;
hipError_t resident_blocks(const void* kernel, int threads, std::atomic<int> (&cache)[kMaxDev], int& out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDev && (out = cache[dev].load(std::memory_order_relaxed)) > 0) return hipSuccess;
    int ncu = 0, per = 0;
    if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, 0)) != hipSuccess) return e;
    out = (per > 0 ? per : 1) * (ncu > 0 ? ncu : 1);
    if (dev >= 0 && dev < kMaxDev) cache[dev].store(out, std::memory_order_relaxed);
    return hipSuccess;
}

template <int VEC, int NW, int L, bool G3>
hipError_t launch_grad(const WkvBwdArgs& A, const BwdGeom& g, bool state, dim3 grid, hipStream_t st) {
    const dim3 block(64 * (NW + 1));
    if (A.r && state) {
        hipLaunchKernelGGL((wkv_bwd_grad_kernel<VEC, NW, L, true, true, G3>), grid, block, 0, st, A, g);
    } else if (A.r) {
        hipLaunchKernelGGL((wkv_bwd_grad_kernel<VEC, NW, L, true, false, G3>), grid, block, 0, st, A, g);
    } else if (state) {
        hipLaunchKernelGGL((wkv_bwd_grad_kernel<VEC, NW, L, false, true, G3>), grid, block, 0, st, A, g);
    } else {
        hipLaunchKernelGGL((wkv_bwd_grad_kernel<VEC, NW, L, false, false, G3>), grid, block, 0, st, A, g);
    }
    return hipGetLastError();
}

template <int VEC, int NW, int L>
hipError_t launch(const WkvBwdArgs& A, const BwdGeom& g, hipStream_t st) {
    const int64_t G = g.B * g.ngrp;
    if (g.nslab > 1) {
        hipError_t e = clear_flags_if_capturing(g.flags_r, G * g.nslab, st);
        if (e == hipSuccess && !g.from_ckpt)
            e = clear_flags_if_capturing(g.flags_c, G * ((g.nslab - 1 + kStateFine - 1) / kStateFine), st);
        if (e != hipSuccess) return e;
    }
    if (g.nslab > 1 && !g.from_ckpt) {
        // Persistent grid: no more workgroups than are resident together.
        const auto kern = wkv_bwd_state_kernel<NW, L>;
        static std::atomic<int> cache[kMaxDev];
        int resident = 0;
        hipError_t e = resident_blocks((const void*)kern, 64 * (kStateFine + 1), cache, resident);
        if (e != hipSuccess) return e;
        const int64_t items = G * ((g.nslab - 1 + kStateFine - 1) / kStateFine);
        const int64_t grid = items < resident ? items : resident;
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * (kStateFine + 1)), 0, st, A, g);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const bool state = A.s_in || A.gs_out || A.gs_in;
    // The 3-D grid numbers blocks x fastest, then y, then z: the flat grid's order.
    const char* flat = std::getenv("LINREC_FLAT_GRID");  // 1: the flat grid at any size (tests)
    const bool g3 = g.B <= 65535 && g.nslab <= 65535 && !(flat && flat[0] == '1');
    if (g3) return launch_grad<VEC, NW, L, true>(A, g, state, dim3((unsigned)g.ngrp, (unsigned)g.B, (unsigned)g.nslab), st);
    return launch_grad<VEC, NW, L, false>(A, g, state, dim3((unsigned)(G * g.nslab)), st);
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
        const int64_t ncoarse = B * ((C + cw - 1) / cw) * ((p.nslab - 1 + kStateFine - 1) / kStateFine);
        bytes += align256((size_t)ncoarse * 8);                            // coarse flags
        bytes += 2 * align256((size_t)(ncoarse * cw) * sizeof(RecordOf<Fwd>::type));  // coarse records
        bytes += align256((size_t)(nrec * cw) * sizeof(FwdRec));           // sums at fine slab ends
        bytes += align256((size_t)nrec * 8);                               // reverse flags
        bytes += 2 * align256((size_t)(nrec * cw) * sizeof(RevRec));       // reverse records
    }
    p.ws_bytes = bytes;
    return p;
}

void wkv_backward_layout(const BwdPlan& p, int64_t B, int64_t C, void* ws, BwdGeom& g) {
    char* at = (char*)ws;
    g.part = reinterpret_cast<double*>(at);
    at += align256((size_t)(B * C) * 2 * sizeof(double));
    g.flags_c = g.flags_r = nullptr;
    g.agg_c = g.incl_c = g.incl_f = g.agg_r = g.incl_r = nullptr;
    if (p.nslab <= 1) return;
    const int64_t cw = 64 * (int64_t)p.vec;
    const int64_t nrec = B * ((C + cw - 1) / cw) * p.nslab;
    const int64_t ncoarse = B * ((C + cw - 1) / cw) * ((p.nslab - 1 + kStateFine - 1) / kStateFine);
    const size_t fl = align256((size_t)nrec * 8);
    const size_t fr = align256((size_t)(nrec * cw) * sizeof(FwdRec));
    const size_t rr = align256((size_t)(nrec * cw) * sizeof(RevRec));
    const size_t cr = align256((size_t)(ncoarse * cw) * sizeof(RecordOf<Fwd>::type));
    g.flags_c = reinterpret_cast<uint64_t*>(at), at += align256((size_t)ncoarse * 8);
    g.agg_c = at, at += cr;
    g.incl_c = at, at += cr;
    g.incl_f = at, at += fr;
    g.flags_r = reinterpret_cast<uint64_t*>(at), at += fl;
    g.agg_r = at, at += rr;
    g.incl_r = at;
}

size_t wkv_backward_ckpt_ws_bytes(int64_t B, int64_t T, int64_t C) {
    const BwdPlan p = wkv_backward_plan(1, B, T, C, 0, 0);
    size_t bytes = align256((size_t)(B * C) * 2 * sizeof(double));  // part
    if (p.nslab > 1) {
        const int64_t nrec = B * ((C + 63) / 64) * p.nslab;
        bytes += align256((size_t)nrec * 8);                          // reverse flags
        bytes += 2 * align256((size_t)(nrec * 64) * sizeof(RevRec));  // reverse records
    }
    return bytes;
}

void wkv_backward_layout_ckpt(const BwdPlan& p, int64_t B, int64_t C, void* ws, const void* ckpt, BwdGeom& g) {
    char* at = (char*)ws;
    g.part = reinterpret_cast<double*>(at);
    at += align256((size_t)(B * C) * 2 * sizeof(double));
    g.flags_c = g.flags_r = nullptr;
    g.agg_c = g.incl_c = g.incl_f = g.agg_r = g.incl_r = nullptr;
    g.from_ckpt = 1;
    if (p.nslab <= 1) return;
    const int64_t nrec = B * ((C + 63) / 64) * p.nslab;
    const size_t rr = align256((size_t)(nrec * 64) * sizeof(RevRec));
    g.incl_f = const_cast<void*>(ckpt);  // read only
    g.flags_r = reinterpret_cast<uint64_t*>(at), at += align256((size_t)nrec * 8);
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

__global__ __launch_bounds__(256) void state_grad_passthrough_kernel(WkvBwdArgs A, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    double f = 0.0, ga = 0.0, gb = 0.0;
    if (A.gs_out) {
        const double p_in = A.s_in ? (double)A.s_in[3 * i + 2] : 0.0;
        f = exp(p_in - (double)A.s_out[3 * i + 2]);
        ga = A.gs_out[2 * i];
        gb = A.gs_out[2 * i + 1];
    }
    A.gs_in[2 * i] = (float)(ga * f);
    A.gs_in[2 * i + 1] = (float)(gb * f);
}

hipError_t run_state_grad_passthrough(const WkvBwdArgs& A, int64_t B, int64_t C, hipStream_t st) {
    const int64_t n = B * C;
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(state_grad_passthrough_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, A, n);
    return hipGetLastError();
}

hipError_t run_zero_wu(float* gw, float* gu, int64_t C, hipStream_t st) {
    hipLaunchKernelGGL(zero_wu_kernel, dim3((unsigned)((C + 255) / 256)), dim3(256), 0, st, gw, gu, C);
    return hipGetLastError();
}

}  // namespace linrec

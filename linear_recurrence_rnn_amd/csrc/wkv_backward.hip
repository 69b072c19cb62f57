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
// One workgroup owns 16 channels of one batch row and the whole sequence, cut in tiles of
// NR chunks of L steps (chunk r of a tile lives in registers of row r):
//   pass F  forward over the tiles: chunk aggregates of (A, B, A', B') -> LDS scan ->
//           the state at every tile start is saved to the workspace (a checkpoint);
//   pass R  tiles from last to first: re-run the forward from the tile's checkpoint (chunked
//           the same way), keeping per step y_t, v_t - y_t, the exponent q_t and g_t/D_t in
//           registers and accumulating the dL/dw, dL/du terms; then scan (G, H) backwards
//           through the tile (chunk aggregates -> reverse LDS scan -> reverse re-run) and
//           write dL/dk, dL/dv.
// The sums are float64 mantissas times 2^p with p an integer exponent (wkv_math.hpp).  The
// gradients are differences of long sums (v G - H, A' - y B'): float64 mantissas keep their
// rounding from accumulating along the sequence; exponentials, reciprocals and the stored
// per-step values stay float32.  On this GPU a float64 FMA issues at the rate of a float32
// FMA without packing.
// dL/dw and dL/du are accumulated per lane in float64, reduced over the rows in a fixed
// order, written per (batch, channel), and summed over the batch by a second kernel: the
// result does not depend on scheduling.
#include "device_common.hpp"
#include "wkv_backward.hpp"
#include "wkv_math.hpp"

namespace linrec {

namespace {

constexpr int kBwdChunk = 8;      // L
constexpr int kBwdRows = 32;      // NR
constexpr int kBwdChannels = 16;  // CW
constexpr int kBwdTile = kBwdChunk * kBwdRows;

// Forward sums over a span: A = a 2^p, B = b 2^p, A' = ad 2^p, B' = bd 2^p.
struct Fwd { double a, b, ad, bd; float p; };
// Reverse sums: G-like = x 2^r, H-like = h 2^r; z 2^r is the sum of the (positive) weights,
// which x and h can cancel below, and sets the exponent.
struct Rev { double x, h, z; float r; };

__device__ __forceinline__ Fwd fwd_identity() { return {0.0, 0.0, 0.0, 0.0, kEmpty}; }
__device__ __forceinline__ Rev rev_identity() { return {0.0, 0.0, 0.0, kEmpty}; }

// State s1, then a span s2 of n2 steps:
//   A = eps^n2 A1 + A2,   A' = eps^n2 (A'1 + n2 A1) + A'2   (B, B' likewise).
__device__ __forceinline__ Fwd fwd_combine(float om, const Fwd& s1, const Fwd& s2, int n2) {
    float p, f1, f2;
    merge_scales(s1.p, (float)s1.b, s2.p, (float)s2.b, mul_split((float)n2, om), p, f1, f2);
    const double g1 = f1, g2 = f2, fn = n2;
    return {fma(s1.a, g1, s2.a * g2), fma(s1.b, g1, s2.b * g2), fma(fma(fn, s1.a, s1.ad), g1, s2.ad * g2),
            fma(fma(fn, s1.b, s1.bd), g1, s2.bd * g2), p};
}

// Reverse sums: s1 is the state at the end of an earlier span s2 of n2 steps; the result is
// the state at the start of s2:  X = s2 + eps^n2 s1.
__device__ __forceinline__ Rev rev_combine(float om, const Rev& s1, const Rev& s2, int n2) {
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

// Inclusive scan over the NR rows of sh (forward direction); tt = steps in the tile.
template <int NR, int CW, int L, int VEC>
__device__ __forceinline__ void fwd_rows_scan(Fwd (&sh)[NR][CW], const float (&om)[VEC], int r, int cl,
                                              int tt) {
#pragma unroll
    for (int d = 1; d < NR; d <<= 1) {
        Fwd tmp[VEC];
        const bool has = r >= d;
        if (has) {
            const int n2 = min((r + 1) * L, tt) - min((r - d + 1) * L, tt);
#pragma unroll
            for (int e = 0; e < VEC; ++e) tmp[e] = fwd_combine(om[e], sh[r - d][cl * VEC + e], sh[r][cl * VEC + e], n2);
        }
        __syncthreads();
        if (has) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) sh[r][cl * VEC + e] = tmp[e];
        }
        __syncthreads();
    }
}

template <int VEC, int CL, int NR, int L>
__global__ __launch_bounds__(CL * NR) void wkv_bwd_kernel(WkvBwdArgs A, int64_t B, int64_t T,
                                                          int64_t C, int64_t ngrp, int64_t ntiles,
                                                          Fwd* __restrict__ ckpt,
                                                          double* __restrict__ part) {
    constexpr int CW = CL * VEC;
    constexpr int TILE = NR * L;
    __shared__ Fwd shf[NR][CW];
    __shared__ Rev shr[NR][CW];
    __shared__ double shacc[NR][CW][2];

    const int tid = threadIdx.x;
    const int r = tid / CL;
    const int cl = tid - r * CL;
    const int64_t lb = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t grp = lb % ngrp;
    const int64_t b = lb / ngrp;
    const int64_t c0 = grp * CW + (int64_t)cl * VEC;
    const bool active = c0 < C;

    float om[VEC], mu[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        om[e] = active ? fminf(A.w[c0 + e] * kLog2e, kMaxOm) : 0.f;
        mu[e] = active ? A.u[c0 + e] * kLog2e : 0.f;
    }

    // ------------------------------ pass F ------------------------------
    Fwd carry[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) carry[e] = fwd_identity();
    for (int64_t i = 0; i < ntiles; ++i) {
        if (r == 0 && active) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) ckpt[(b * ntiles + i) * C + c0 + e] = carry[e];
        }
        const int64_t t0 = i * TILE;
        const int tt = (int)min((int64_t)TILE, T - t0);
        const int n = active ? max(0, min(L, tt - r * L)) : 0;
        const int64_t off = (b * T + t0 + (int64_t)r * L) * C + c0;
        float kk[L][VEC], vv[L][VEC];
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                const FV<VEC> kt = ldg<VEC>(A.k + off + (int64_t)j * C);
                const FV<VEC> vt = ldg<VEC>(A.v + off + (int64_t)j * C);
#pragma unroll
                for (int e = 0; e < VEC; ++e) { kk[j][e] = kt.v[e] * kLog2e; vv[j][e] = vt.v[e]; }
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e) { kk[j][e] = 0.f; vv[j][e] = 0.f; }
            }
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) shf[r][cl * VEC + e] = fwd_chunk<L, VEC>(om[e], kk, vv, e, n);
        __syncthreads();
        fwd_rows_scan<NR, CW, L, VEC>(shf, om, r, cl, tt);
#pragma unroll
        for (int e = 0; e < VEC; ++e) carry[e] = fwd_combine(om[e], carry[e], shf[NR - 1][cl * VEC + e], tt);
        __syncthreads();
    }

    // ------------------------------ pass R ------------------------------
    Rev rcarry[VEC];
    double accw[VEC], accu[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        rcarry[e] = rev_identity();
        accw[e] = 0.0;
        accu[e] = 0.0;
    }
    for (int64_t i = ntiles - 1; i >= 0; --i) {
        const int64_t t0 = i * TILE;
        const int tt = (int)min((int64_t)TILE, T - t0);
        const int n = active ? max(0, min(L, tt - r * L)) : 0;
        const int64_t off = (b * T + t0 + (int64_t)r * L) * C + c0;
        float kk[L][VEC], vv[L][VEC], gg[L][VEC];
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                const FV<VEC> kt = ldg<VEC>(A.k + off + (int64_t)j * C);
                const FV<VEC> vt = ldg<VEC>(A.v + off + (int64_t)j * C);
                const FV<VEC> gt = ldg<VEC>(A.gy + off + (int64_t)j * C);
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    kk[j][e] = kt.v[e] * kLog2e;
                    vv[j][e] = vt.v[e];
                    gg[j][e] = gt.v[e];
                }
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e) { kk[j][e] = 0.f; vv[j][e] = 0.f; gg[j][e] = 0.f; }
            }
        }
        Fwd tin[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) tin[e] = active ? ckpt[(b * ntiles + i) * C + c0 + e] : fwd_identity();

        // Forward phases 1 and 2 (as in pass F).
#pragma unroll
        for (int e = 0; e < VEC; ++e) shf[r][cl * VEC + e] = fwd_chunk<L, VEC>(om[e], kk, vv, e, n);
        __syncthreads();
        fwd_rows_scan<NR, CW, L, VEC>(shf, om, r, cl, tt);

        // Forward phase 3: per step y, v - y, the exponent q and g/dm; dL/dw, dL/du terms.
        float cg[L][VEC], qs[L][VEC], ys[L][VEC], dv[L][VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            Fwd s = (r == 0) ? tin[e]
                             : fwd_combine(om[e], tin[e], shf[r - 1][cl * VEC + e], min(r * L, tt));
            double sw = 0.0, su = 0.0;
#pragma unroll
            for (int j = 0; j < L; ++j) {
                if (j < n) {
                    const float kj = kk[j][e];
                    const double vj = vv[j][e];
                    const float M = mag(s.p, (float)s.b);
                    const float q = ceilf(fmaxf(M, kj + mu[e]));
                    const float e1 = fast_exp2(s.p - q), e2 = fast_exp2((kj - q) + mu[e]);
                    const double dm = fma(s.b, (double)e1, (double)e2);  // D_t = dm 2^q
                    const float inv = __builtin_amdgcn_rcpf((float)dm);
                    const float y = (float)fma(s.a, (double)e1, vj * e2) * inv;
                    const float vmy = e1 * (float)fma(vj, s.b, -s.a) * inv;  // v_t - y_t
                    const float c = gg[j][e] * inv;
                    sw -= (double)(c * e1) * fma(-(double)y, s.bd, s.ad);
                    su += (double)(c * e2 * vmy);
                    cg[j][e] = c;
                    qs[j][e] = q;
                    ys[j][e] = y;
                    dv[j][e] = vmy;
                    const float q2 = ceilf(fmaxf(M - om[e], kj));
                    const double f1 = fast_exp2((s.p - q2) - om[e]), f2 = fast_exp2(kj - q2);
                    s.ad = (s.ad + s.a) * f1;
                    s.bd = (s.bd + s.b) * f1;
                    s.a = fma(s.a, f1, vj * f2);
                    s.b = fma(s.b, f1, f2);
                    s.p = q2;
                } else {
                    cg[j][e] = 0.f;
                    qs[j][e] = 0.f;
                    ys[j][e] = 0.f;
                    dv[j][e] = 0.f;
                }
            }
            accw[e] += sw;
            accu[e] += su;
        }

        // Reverse phase 1: (G, H) sums of my chunk seen from its first step, weights
        // 2^{-q_j - j om}.
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            Rev s = rev_identity();
            if (n > 0) {
                float m[L];
                float mx = kEmpty;
#pragma unroll
                for (int j = 0; j < L; ++j) {
                    m[j] = (j < n) ? fmaf(-(float)j, om[e], -qs[j][e]) : kEmpty;
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
            }
            shr[r][cl * VEC + e] = s;
        }
        __syncthreads();
        // Reverse phase 2: suffix scan over the rows.  start(x) = steps before chunk x.
        auto start_of = [&](int x) { return min(x * L, tt); };
#pragma unroll
        for (int d = 1; d < NR; d <<= 1) {
            Rev tmp[VEC];
            const bool has = r + d < NR;
            if (has) {
                const int n2 = start_of(r + d) - start_of(r);
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    tmp[e] = rev_combine(om[e], shr[r + d][cl * VEC + e], shr[r][cl * VEC + e], n2);
            }
            __syncthreads();
            if (has) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) shr[r][cl * VEC + e] = tmp[e];
            }
            __syncthreads();
        }

        // Reverse phase 3: walk my chunk backwards from the state at its end.
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            Rev s = (r == NR - 1) ? rcarry[e]
                                  : rev_combine(om[e], rcarry[e], shr[r + 1][cl * VEC + e], tt - start_of(r + 1));
#pragma unroll
            for (int j = L - 1; j >= 0; --j) {
                if (j < n) {
                    const float sc = fast_exp2(s.r + kk[j][e]);                            // alpha_s scale
                    const float dgv = cg[j][e] * fast_exp2((kk[j][e] - qs[j][e]) + mu[e]);  // g beta / D
                    const float gvv = (float)fma(s.x, (double)sc, (double)dgv);
                    const float gkk = fmaf(dgv, dv[j][e], sc * (float)fma((double)vv[j][e], s.x, -s.h));
                    kk[j][e] = gkk;  // registers reused for the outputs
                    vv[j][e] = gvv;
                    const float r2 = ceilf(fmaxf(mag(s.r, (float)s.z) - om[e], -qs[j][e]));
                    const double f1 = fast_exp2((s.r - r2) - om[e]);
                    const float w2 = fast_exp2(-qs[j][e] - r2);
                    const double f2 = w2 * cg[j][e];
                    s.x = fma(s.x, f1, f2);
                    s.h = fma(s.h, f1, f2 * ys[j][e]);
                    s.z = fma(s.z, f1, (double)w2);
                    s.r = r2;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) {
                FV<VEC> ok, ov;
#pragma unroll
                for (int e = 0; e < VEC; ++e) { ok.v[e] = kk[j][e]; ov.v[e] = vv[j][e]; }
                stg<VEC>(A.gk + off + (int64_t)j * C, ok);
                stg<VEC>(A.gv + off + (int64_t)j * C, ov);
            }
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) rcarry[e] = rev_combine(om[e], rcarry[e], shr[0][cl * VEC + e], tt);
        __syncthreads();
    }

    // dL/dw, dL/du of this (batch row, channel): rows summed in order.
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        shacc[r][cl * VEC + e][0] = accw[e];
        shacc[r][cl * VEC + e][1] = accu[e];
    }
    __syncthreads();
    if (r == 0 && active) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            double sw = 0.0, su = 0.0;
            for (int x = 0; x < NR; ++x) {
                sw += shacc[x][cl * VEC + e][0];
                su += shacc[x][cl * VEC + e][1];
            }
            part[2 * (b * C + c0 + e)] = sw;
            part[2 * (b * C + c0 + e) + 1] = su;
        }
    }
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

}  // namespace

BwdPlan wkv_backward_plan(int64_t B, int64_t T, int64_t C) {
    BwdPlan p{};
    p.vec = 1;
    p.ntiles = (T + kBwdTile - 1) / kBwdTile;
    p.ckpt_bytes = align256((size_t)(B * p.ntiles * C) * sizeof(Fwd));
    p.ws_bytes = p.ckpt_bytes + align256((size_t)(B * C) * 2 * sizeof(double));
    return p;
}

hipError_t run_wkv_backward(const WkvBwdArgs& A, int64_t B, int64_t T, int64_t C, const BwdPlan& p,
                            void* ws, hipStream_t st) {
    const int64_t ngrp = (C + kBwdChannels - 1) / kBwdChannels;
    Fwd* ckpt = reinterpret_cast<Fwd*>(ws);
    double* part = reinterpret_cast<double*>((char*)ws + p.ckpt_bytes);
    const dim3 grid((unsigned)(B * ngrp));
    if (p.vec == 2) {
        constexpr int CL = kBwdChannels / 2;
        hipLaunchKernelGGL((wkv_bwd_kernel<2, CL, kBwdRows, kBwdChunk>), grid, dim3(CL * kBwdRows), 0, st,
                           A, B, T, C, ngrp, p.ntiles, ckpt, part);
    } else {
        constexpr int CL = kBwdChannels;
        hipLaunchKernelGGL((wkv_bwd_kernel<1, CL, kBwdRows, kBwdChunk>), grid, dim3(CL * kBwdRows), 0, st,
                           A, B, T, C, ngrp, p.ntiles, ckpt, part);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(wkv_bwd_wu_kernel, dim3((unsigned)((C + 255) / 256)), dim3(256), 0, st, part, B, C,
                       A.gw, A.gu);
    return hipGetLastError();
}

hipError_t run_zero_wu(float* gw, float* gu, int64_t C, hipStream_t st) {
    hipLaunchKernelGGL(zero_wu_kernel, dim3((unsigned)((C + 255) / 256)), dim3(256), 0, st, gw, gu, C);
    return hipGetLastError();
}

}  // namespace linrec

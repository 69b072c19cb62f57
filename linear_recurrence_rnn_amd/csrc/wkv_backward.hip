// wkv_backward.hip -- WKV-4 backward on gfx950.
//
// Chain rule of eq. (14) of the RWKV-LLM page ("Time-mixing block"); the pages give no
// backward.  With eps = e^{-w}, alpha_i = e^{k_i}, beta_t = e^{u+k_t}, D_t = B_t + beta_t,
//   dL/du   = sum_t g_t beta_t (v_t - y_t) / D_t
//   dL/dw   = -sum_t g_t (A'_t - y_t B'_t) / D_t,   A'_t = sum_{i<t} (t-1-i) eps^{t-1-i} alpha_i v_i
//   dL/dv_s = g_s beta_s / D_s + alpha_s G_s,       G_s = sum_{t>s} eps^{t-1-s} g_t / D_t
//   dL/dk_s = g_s beta_s (v_s - y_s) / D_s + alpha_s (v_s G_s - H_s),  H_s likewise with g_t y_t
//
// One workgroup owns 16 channels of one batch row and the whole sequence, cut in tiles of
// NR chunks of L steps (chunk r of a tile lives in registers of row r):
//   pass F  forward over the tiles: chunk aggregates of (A, B, A', B') -> LDS scan ->
//           the state at every tile start is saved to the workspace (a checkpoint);
//   pass R  tiles from last to first: re-run the forward from the tile's checkpoint (chunked
//           the same way), keeping y_t, the scale q_t and g_t/D_t per step in registers and
//           accumulating the dL/dw, dL/du terms; then scan (G, H) backwards through the tile
//           (chunk aggregates -> reverse LDS scan -> reverse re-run) and write dL/dk, dL/dv.
// All sums are kept in base-2 scaled form (value = mantissa * 2^scale, scale the running
// maximum exponent), so no exponential with a positive argument is ever formed.
// dL/dw and dL/du are accumulated per lane in float64, reduced over the rows in a fixed
// order, written per (batch, channel), and summed over the batch by a second kernel: the
// result does not depend on scheduling.
#include "device_common.hpp"
#include "wkv_backward.hpp"

namespace linrec {

namespace {

constexpr int kBwdChunk = 8;      // L
constexpr int kBwdRows = 32;      // NR
constexpr int kBwdChannels = 16;  // CW
constexpr int kBwdTile = kBwdChunk * kBwdRows;

// Forward state over a span: A = a 2^p, B = b 2^p, A' = ad 2^p, B' = bd 2^p.
struct Fwd5 { float a, b, ad, bd, p; };
// Reverse state: G-like sum = x 2^r, H-like sum = h 2^r.
struct Rev3 { float x, h, r; };

__device__ __forceinline__ Fwd5 fwd_identity() { return {0.f, 0.f, 0.f, 0.f, kEmpty}; }
__device__ __forceinline__ Rev3 rev_identity() { return {0.f, 0.f, kEmpty}; }

// State s1, then a span s2 of n2 steps:
//   A = eps^n2 A1 + A2,   A' = eps^n2 (A'1 + n2 A1) + A'2   (B, B' likewise).
__device__ __forceinline__ Fwd5 fwd_combine(float om, const Fwd5& s1, const Fwd5& s2, int n2) {
    const float p1 = fmaxf(s1.p - (float)n2 * om, kEmpty);
    const float p = fmaxf(p1, s2.p);
    const float f1 = fast_exp2(p1 - p), f2 = fast_exp2(s2.p - p);
    const float fn = (float)n2;
    Fwd5 r;
    r.a = fmaf(s1.a, f1, s2.a * f2);
    r.b = fmaf(s1.b, f1, s2.b * f2);
    r.ad = fmaf(fmaf(fn, s1.a, s1.ad), f1, s2.ad * f2);
    r.bd = fmaf(fmaf(fn, s1.b, s1.bd), f1, s2.bd * f2);
    r.p = p;
    return r;
}

// Reverse sums: s1 is the state at the end of an earlier span s2 of n2 steps; the result is
// the state at the start of s2:  X = s2 + eps^n2 s1.
__device__ __forceinline__ Rev3 rev_combine(float om, const Rev3& s1, const Rev3& s2, int n2) {
    const float r1 = fmaxf(s1.r - (float)n2 * om, kEmpty);
    const float r = fmaxf(r1, s2.r);
    const float f1 = fast_exp2(r1 - r), f2 = fast_exp2(s2.r - r);
    return {fmaf(s1.x, f1, s2.x * f2), fmaf(s1.h, f1, s2.h * f2), r};
}

template <int VEC, int CL, int NR, int L>
__global__ __launch_bounds__(CL * NR) void wkv_bwd_kernel(WkvBwdArgs A, int64_t B, int64_t T,
                                                          int64_t C, int64_t ngrp, int64_t ntiles,
                                                          Fwd5* __restrict__ ckpt,
                                                          double* __restrict__ part) {
    constexpr int CW = CL * VEC;
    constexpr int TILE = NR * L;
    __shared__ Fwd5 shf[NR][CW];
    __shared__ Rev3 shr[NR][CW];
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
        om[e] = active ? A.w[c0 + e] * kLog2e : 0.f;
        mu[e] = active ? A.u[c0 + e] * kLog2e : 0.f;
    }
    auto end_of = [&](int x, int tt) { return min((x + 1) * L, tt); };

    // ------------------------------ pass F ------------------------------
    Fwd5 carry[VEC];
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
        // Phase 1: (A, B, A', B') of my chunk from the empty state.
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            Fwd5 s = fwd_identity();
            if (n > 0) {
                float p = kEmpty;
                float m[L];
#pragma unroll
                for (int j = 0; j < L; ++j) {
                    m[j] = (j < n) ? fmaf(-(float)(n - 1 - j), om[e], kk[j][e]) : kEmpty;
                    p = fmaxf(p, m[j]);
                }
                s.p = p;
#pragma unroll
                for (int j = 0; j < L; ++j) {
                    const float f = fast_exp2(m[j] - p);
                    const float fd = (j < n) ? f * (float)(n - 1 - j) : 0.f;
                    s.a = fmaf(f, vv[j][e], s.a);
                    s.b += f;
                    s.ad = fmaf(fd, vv[j][e], s.ad);
                    s.bd += fd;
                }
            }
            shf[r][cl * VEC + e] = s;
        }
        __syncthreads();
        // Phase 2: inclusive scan over the rows.
#pragma unroll
        for (int d = 1; d < NR; d <<= 1) {
            Fwd5 tmp[VEC];
            const bool has = r >= d;
            if (has) {
                const int n2 = end_of(r, tt) - end_of(r - d, tt);
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    tmp[e] = fwd_combine(om[e], shf[r - d][cl * VEC + e], shf[r][cl * VEC + e], n2);
            }
            __syncthreads();
            if (has) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) shf[r][cl * VEC + e] = tmp[e];
            }
            __syncthreads();
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) carry[e] = fwd_combine(om[e], carry[e], shf[NR - 1][cl * VEC + e], tt);
        __syncthreads();
    }

    // ------------------------------ pass R ------------------------------
    Rev3 rcarry[VEC];
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
        Fwd5 tin[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            tin[e] = active ? ckpt[(b * ntiles + i) * C + c0 + e] : fwd_identity();

        // Forward phase 1 + 2 (as in pass F).
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            Fwd5 s = fwd_identity();
            if (n > 0) {
                float p = kEmpty;
                float m[L];
#pragma unroll
                for (int j = 0; j < L; ++j) {
                    m[j] = (j < n) ? fmaf(-(float)(n - 1 - j), om[e], kk[j][e]) : kEmpty;
                    p = fmaxf(p, m[j]);
                }
                s.p = p;
#pragma unroll
                for (int j = 0; j < L; ++j) {
                    const float f = fast_exp2(m[j] - p);
                    const float fd = (j < n) ? f * (float)(n - 1 - j) : 0.f;
                    s.a = fmaf(f, vv[j][e], s.a);
                    s.b += f;
                    s.ad = fmaf(fd, vv[j][e], s.ad);
                    s.bd += fd;
                }
            }
            shf[r][cl * VEC + e] = s;
        }
        __syncthreads();
#pragma unroll
        for (int d = 1; d < NR; d <<= 1) {
            Fwd5 tmp[VEC];
            const bool has = r >= d;
            if (has) {
                const int n2 = end_of(r, tt) - end_of(r - d, tt);
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    tmp[e] = fwd_combine(om[e], shf[r - d][cl * VEC + e], shf[r][cl * VEC + e], n2);
            }
            __syncthreads();
            if (has) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) shf[r][cl * VEC + e] = tmp[e];
            }
            __syncthreads();
        }

        // Forward phase 3: per-step y, scale q and g/Dm; dL/dw and dL/du terms.
        float cg[L][VEC], qs[L][VEC], ys[L][VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            Fwd5 s = (r == 0) ? tin[e] : fwd_combine(om[e], tin[e], shf[r - 1][cl * VEC + e], end_of(r - 1, tt));
            float sw = 0.f, su = 0.f;
#pragma unroll
            for (int j = 0; j < L; ++j) {
                if (j < n) {
                    const float ww = mu[e] + kk[j][e];
                    const float q = fmaxf(s.p, ww);
                    const float e1 = fast_exp2(s.p - q), e2 = fast_exp2(ww - q);
                    const float dm = fmaf(s.b, e1, e2);  // D_t = dm 2^q, dm >= 1
                    const float inv = __builtin_amdgcn_rcpf(dm);
                    const float y = fmaf(s.a, e1, vv[j][e] * e2) * inv;
                    const float c = gg[j][e] * inv;
                    sw = fmaf(-c * e1, fmaf(-y, s.bd, s.ad), sw);
                    su = fmaf(c * e2, vv[j][e] - y, su);
                    cg[j][e] = c;
                    qs[j][e] = q;
                    ys[j][e] = y;
                    const float pw = s.p - om[e];
                    const float q2 = fmaxf(pw, kk[j][e]);
                    const float f1 = fast_exp2(pw - q2), f2 = fast_exp2(kk[j][e] - q2);
                    s.ad = (s.ad + s.a) * f1;
                    s.bd = (s.bd + s.b) * f1;
                    s.a = fmaf(s.a, f1, vv[j][e] * f2);
                    s.b = fmaf(s.b, f1, f2);
                    s.p = q2;
                } else {
                    cg[j][e] = 0.f;
                    qs[j][e] = 0.f;
                    ys[j][e] = 0.f;
                }
            }
            accw[e] += (double)sw;
            accu[e] += (double)su;
        }

        // Reverse phase 1: (G, H) sums of my chunk seen from its first step.
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            Rev3 s = rev_identity();
            if (n > 0) {
                float m[L];
                float rr = kEmpty;
#pragma unroll
                for (int j = 0; j < L; ++j) {
                    m[j] = (j < n) ? fmaf(-(float)j, om[e], -qs[j][e]) : kEmpty;
                    rr = fmaxf(rr, m[j]);
                }
                s.r = rr;
#pragma unroll
                for (int j = 0; j < L; ++j) {
                    const float f = fast_exp2(m[j] - rr) * cg[j][e];
                    s.x += f;
                    s.h = fmaf(f, ys[j][e], s.h);
                }
            }
            shr[r][cl * VEC + e] = s;
        }
        __syncthreads();
        // Reverse phase 2: suffix scan over the rows.  start(x) = steps before chunk x.
        auto start_of = [&](int x) { return min(x * L, tt); };
#pragma unroll
        for (int d = 1; d < NR; d <<= 1) {
            Rev3 tmp[VEC];
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
            Rev3 s = (r == NR - 1) ? rcarry[e]
                                   : rev_combine(om[e], rcarry[e], shr[r + 1][cl * VEC + e],
                                                 tt - start_of(r + 1));
#pragma unroll
            for (int j = L - 1; j >= 0; --j) {
                if (j < n) {
                    const float sc = fast_exp2(s.r + kk[j][e]);                     // alpha_s scale
                    const float dgv = cg[j][e] * fast_exp2(mu[e] + kk[j][e] - qs[j][e]);  // g beta / D
                    const float gvv = fmaf(s.x, sc, dgv);
                    const float gkk = fmaf(dgv, vv[j][e] - ys[j][e], sc * fmaf(vv[j][e], s.x, -s.h));
                    kk[j][e] = gkk;  // registers reused for the outputs
                    vv[j][e] = gvv;
                    const float rw = s.r - om[e];
                    const float r2 = fmaxf(rw, -qs[j][e]);
                    const float f1 = fast_exp2(rw - r2), f2 = fast_exp2(-qs[j][e] - r2) * cg[j][e];
                    s.x = fmaf(s.x, f1, f2);
                    s.h = fmaf(s.h, f1, f2 * ys[j][e]);
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
    p.ckpt_bytes = align256((size_t)(B * p.ntiles * C) * sizeof(Fwd5));
    p.ws_bytes = p.ckpt_bytes + align256((size_t)(B * C) * 2 * sizeof(double));
    return p;
}

hipError_t run_wkv_backward(const WkvBwdArgs& A, int64_t B, int64_t T, int64_t C, const BwdPlan& p,
                            void* ws, hipStream_t st) {
    const int64_t ngrp = (C + kBwdChannels - 1) / kBwdChannels;
    Fwd5* ckpt = reinterpret_cast<Fwd5*>(ws);
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

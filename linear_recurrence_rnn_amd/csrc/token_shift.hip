// token_shift.hip -- the token shift of the RWKV time-mix block on gfx950.
//
// RWKV-LLM page, section "Time-mixing block", eqs. (11)-(13): the inputs of the r, k and v
// projections interpolate per channel between the current token and the previous one,
//   out[m,b,t,c] = mu[m,c] x[b,t,c] + (1 - mu[m,c]) x[b,t-1,c] = p + mu (x - p),  p = x[b,t-1,c],
// with x[b,-1,c] = x_prev[b,c] (the last token of an earlier call) or 0.  One pass reads x
// once and writes all M mixes (the r, k, v inputs of the time mix, or the r, k inputs of the
// channel mix), instead of one pass per mix.
//
// Backward (chain rule; the pages give none), with g = dL/dout:
//   gx[b,t,c]    = sum_m mu[m,c] g[m,b,t,c] + (1 - mu[m,c]) g[m,b,t+1,c]
//   gx_prev[b,c] = sum_m (1 - mu[m,c]) g[m,b,0,c]
//   gmu[m,c]     = sum_{b,t} g[m,b,t,c] (x[b,t,c] - x[b,t-1,c])
//
// Layout of work: a wave owns VEC channels per lane (64 * VEC contiguous channels, so every
// wave-wide access is one contiguous row segment) over TS consecutive time steps, and holds
// the rows it needs in registers: the TS rows of its span and the row before it (read
// again by the neighbouring span, 1/TS extra), plus, in the backward, the row after it
// (there handed over between the waves of a block, so 1/(8 TS) extra).
// Both passes are HBM-bound streams (forward 4 + 4M bytes per element, backward 8 + 4M).
// gmu is summed in float64: per wave over its span, over the 8 waves of a backward block in
// order, then over blocks in a fixed order by a second kernel, so it does not depend on
// scheduling.
#include "device_common.hpp"
#include "token_shift.hpp"

namespace linrec {

namespace {

constexpr int kShiftTS = 16;       // time steps per wave
constexpr int kShiftWaves = 4;     // waves per block

template <int VEC>
__device__ __forceinline__ FV<VEC> load_or_zero(const float* p, bool ok) {
    FV<VEC> r{};
    if (ok) r = ldg<VEC>(p);
    return r;
}

// Forward: wave item (b, tc, grp), grp fastest, so neighbouring waves stream neighbouring
// channel groups of the same rows.
template <int VEC>
__global__ __launch_bounds__(64 * kShiftWaves) void token_shift_kernel(TokenShiftArgs A, int64_t B, int64_t T,
                                                                       int64_t C, int M) {
    constexpr int TS = kShiftTS;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t ngrp = (C + 64 * VEC - 1) / (64 * VEC), ntc = (T + TS - 1) / TS;
    const int64_t item = (int64_t)blockIdx.x * kShiftWaves + wv;
    if (item >= B * ntc * ngrp) return;  // wave-uniform
    const int64_t grp = item % ngrp, tc = (item / ngrp) % ntc, b = item / (ngrp * ntc);
    const int64_t c = grp * 64 * VEC + (int64_t)lane * VEC;
    const bool active = c < C;  // C is a multiple of VEC
    const int64_t t0 = tc * TS;
    const int n = (int)((T - t0) < TS ? (T - t0) : TS);
    const float* xr = A.x + (b * T + t0) * C + c;

    FV<VEC> prev = load_or_zero<VEC>(t0 > 0 ? xr - C : (A.x_prev ? A.x_prev + b * C + c : nullptr),
                                     active && (t0 > 0 || A.x_prev));
    FV<VEC> xs[TS];
#pragma unroll
    for (int j = 0; j < TS; ++j) xs[j] = load_or_zero<VEC>(xr + (int64_t)j * C, active && j < n);
    if (!active) return;
    for (int m = 0; m < M; ++m) {
        float mu[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) mu[e] = A.mu[m * C + c + e];
        float* o = A.out + (int64_t)m * B * T * C + (b * T + t0) * C + c;
        FV<VEC> p = prev;
#pragma unroll
        for (int j = 0; j < TS; ++j) {
            if (j < n) {
                FV<VEC> y;
#pragma unroll
                for (int e = 0; e < VEC; ++e) y.v[e] = fmaf(mu[e], xs[j].v[e] - p.v[e], p.v[e]);
                stg<VEC>(o + (int64_t)j * C, y);
            }
            p = xs[j];
        }
    }
}

// Backward: block (b, tcb, grp) of kShiftBwdWaves waves; wave w takes steps
// [(tcb*NWV + w)*TS, +TS).  Every row the wave needs (x and all M gradients) is loaded before
// any is used, so the whole span is in flight.  The rows a span needs beyond its own -- x
// at t0-1 and the gradients at t0+TS -- are the neighbouring waves' last and first rows,
// handed over through LDS; only the block's outer waves read them from memory.
constexpr int kShiftBwdWaves = 8;

template <int VEC, int TS, int M>
__global__ __launch_bounds__(64 * kShiftBwdWaves) void token_shift_bwd_kernel(TokenShiftBwdArgs A, int64_t B,
                                                                              int64_t T, int64_t C) {
    constexpr int CW = 64 * VEC;
    constexpr int NWV = kShiftBwdWaves;
    __shared__ double sh[NWV][M][CW];    // the waves' dL/dmu sums
    __shared__ float sh_xl[NWV][CW];     // each span's last x row
    __shared__ float sh_gf[NWV][M][CW];  // each span's first gradient rows
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t ngrp = (C + CW - 1) / CW, ntcb = (T + NWV * TS - 1) / (NWV * TS);
    const int64_t blk = blockIdx.x;
    const int64_t grp = blk % ngrp, tcb = (blk / ngrp) % ntcb, b = blk / (ngrp * ntcb);
    const int64_t c = grp * CW + (int64_t)lane * VEC;
    const bool active = c < C;
    const int64_t t0 = (tcb * NWV + wv) * TS;
    const int n = t0 >= T ? 0 : (int)((T - t0) < TS ? (T - t0) : TS);
    const float* xr = A.x + (b * T + t0) * C + c;

    // x rows t0-1 .. t0+n-1 and g rows t0 .. t0+n (0 past the end of the sequence).  Row
    // t0-1 is x_prev, or 0, at the start of the sequence.
    FV<VEC> xs[TS + 1];
    if (wv == 0)
        xs[0] = load_or_zero<VEC>(t0 > 0 ? xr - C : (A.x_prev ? A.x_prev + b * C + c : nullptr),
                                  active && n > 0 && (t0 > 0 || A.x_prev));
#pragma unroll
    for (int j = 0; j < TS; ++j) xs[j + 1] = load_or_zero<VEC>(xr + (int64_t)j * C, active && j < n);
    FV<VEC> gs[M][TS + 1];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const float* gr = A.g + (int64_t)m * B * T * C + (b * T + t0) * C + c;
#pragma unroll
        for (int j = 0; j < TS; ++j) gs[m][j] = load_or_zero<VEC>(gr + (int64_t)j * C, active && j < n);
        if (wv == NWV - 1) gs[m][TS] = load_or_zero<VEC>(gr + (int64_t)TS * C, active && n == TS && t0 + TS < T);
    }
    // Hand the neighbours their rows: a span's last x row (row t0+TS-1 when the span is
    // full; the next span is empty otherwise) and its first gradient rows (0 when n = 0).
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        sh_xl[wv][lane * VEC + e] = xs[TS].v[e];
#pragma unroll
        for (int m = 0; m < M; ++m) sh_gf[wv][m][lane * VEC + e] = gs[m][0].v[e];
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        if (wv > 0) xs[0].v[e] = sh_xl[wv - 1][lane * VEC + e];
#pragma unroll
        for (int m = 0; m < M; ++m)
            if (wv < NWV - 1) gs[m][TS].v[e] = n == TS ? sh_gf[wv + 1][m][lane * VEC + e] : 0.f;
    }
    float mu[M][VEC];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int e = 0; e < VEC; ++e) mu[m][e] = active ? A.mu[m * C + c + e] : 0.f;

    float gxp[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) gxp[e] = 0.f;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        double part[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            part[e] = 0.0;
#pragma unroll
            for (int j = 0; j < TS; ++j)
                if (j < n) part[e] = fma((double)gs[m][j].v[e], (double)xs[j + 1].v[e] - (double)xs[j].v[e], part[e]);
            gxp[e] = fmaf(1.f - mu[m][e], gs[m][0].v[e], gxp[e]);
            sh[wv][m][lane * VEC + e] = part[e];
        }
    }
    if (active) {
        float* go = A.gx + (b * T + t0) * C + c;
#pragma unroll
        for (int j = 0; j < TS; ++j) {
            if (j < n) {
                FV<VEC> gx;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    float acc = 0.f;
#pragma unroll
                    for (int m = 0; m < M; ++m)
                        acc = fmaf(mu[m][e], gs[m][j].v[e], fmaf(1.f - mu[m][e], gs[m][j + 1].v[e], acc));
                    gx.v[e] = acc;
                }
                stg<VEC>(go + (int64_t)j * C, gx);
            }
        }
        if (t0 == 0 && n > 0 && A.gx_prev) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) A.gx_prev[b * C + c + e] = gxp[e];
        }
    }
    __syncthreads();
    if (wv == 0 && active) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                double s = 0.0;
                for (int w = 0; w < NWV; ++w) s += sh[w][m][lane * VEC + e];
                A.part[((b * ntcb + tcb) * M + m) * C + c + e] = s;
            }
        }
    }
}

// gmu[m,c] = sum over the nblk block sums (b outer, tcb inner), in a fixed association:
// block (m, 64 channels) of 16 waves; wave w adds the w-th sixteenth of the block sums
// round-robin into 8 accumulators (8 loads in flight at a time), which are then added in
// order, and the 16 parts are added in order.
constexpr int kMuWaves = 16;

__global__ __launch_bounds__(64 * kMuWaves) void token_shift_mu_kernel(TokenShiftBwdArgs A, int64_t nblk, int64_t C,
                                                                        int M) {
    __shared__ double sh[kMuWaves][64];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int64_t ncg = (C + 63) / 64;
    const int64_t m = blockIdx.x / ncg, c = (blockIdx.x - m * ncg) * 64 + lane;
    const int64_t q = (nblk + kMuWaves - 1) / kMuWaves;
    const int64_t k0 = wv * q < nblk ? wv * q : nblk, k1 = (k0 + q) < nblk ? (k0 + q) : nblk;
    double acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0;
    if (c < C) {
        int64_t k = k0;
        for (; k + 8 <= k1; k += 8) {
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += A.part[((k + i) * M + m) * C + c];
        }
        for (int i = 0; k < k1; ++k, ++i) acc[i] += A.part[(k * M + m) * C + c];
    }
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += acc[i];
    sh[wv][lane] = s;
    __syncthreads();
    if (wv == 0 && c < C) {
        double t = 0.0;
        for (int w = 0; w < kMuWaves; ++w) t += sh[w][lane];
        A.gmu[m * C + c] = (float)t;
    }
}

}  // namespace

hipError_t run_token_shift(const TokenShiftArgs& A, int64_t B, int64_t T, int64_t C, int M, int vec,
                           hipStream_t st) {
    const int64_t cw = 64 * vec;
    const int64_t items = B * ((T + kShiftTS - 1) / kShiftTS) * ((C + cw - 1) / cw);
    const dim3 grid((unsigned)((items + kShiftWaves - 1) / kShiftWaves)), block(64 * kShiftWaves);
    if (vec == 4) hipLaunchKernelGGL(token_shift_kernel<4>, grid, block, 0, st, A, B, T, C, M);
    else if (vec == 2) hipLaunchKernelGGL(token_shift_kernel<2>, grid, block, 0, st, A, B, T, C, M);
    else hipLaunchKernelGGL(token_shift_kernel<1>, grid, block, 0, st, A, B, T, C, M);
    return hipGetLastError();
}

// Backward spans: 16 steps for one channel per lane, 4 for two (the gradient rows of every
// mix stay in registers).  With two channels per lane, 4-step spans hold 66 VGPRs, so three
// 8-wave blocks share a CU (B8 T1024 C768, 3 mixes: 30.9 -> 30.3 us with the dL/dmu sum);
// 8-step spans held 106 (two blocks per CU), 6-step spans ran 34.9 us (ragged blocks), and
// capping 8-step spans at 80 VGPRs spilled (56.2 us).
constexpr int shift_bwd_ts(int vec) { return vec == 2 ? 4 : kShiftTS; }

size_t token_shift_backward_ws_bytes(int64_t B, int64_t T, int64_t C, int M, int vec) {
    const int ts = shift_bwd_ts(vec);
    const int64_t ntcb = (T + kShiftBwdWaves * ts - 1) / (kShiftBwdWaves * ts);
    return (size_t)(B * ntcb * M * C) * sizeof(double);
}

namespace {
template <int VEC, int TS>
void launch_bwd(const TokenShiftBwdArgs& A, dim3 grid, int64_t B, int64_t T, int64_t C, int M, hipStream_t st) {
    const dim3 block(64 * kShiftBwdWaves);
    if (M == 1) hipLaunchKernelGGL((token_shift_bwd_kernel<VEC, TS, 1>), grid, block, 0, st, A, B, T, C);
    else if (M == 2) hipLaunchKernelGGL((token_shift_bwd_kernel<VEC, TS, 2>), grid, block, 0, st, A, B, T, C);
    else if (M == 3) hipLaunchKernelGGL((token_shift_bwd_kernel<VEC, TS, 3>), grid, block, 0, st, A, B, T, C);
    else hipLaunchKernelGGL((token_shift_bwd_kernel<VEC, TS, 4>), grid, block, 0, st, A, B, T, C);
}
}  // namespace

hipError_t run_token_shift_backward(const TokenShiftBwdArgs& A, int64_t B, int64_t T, int64_t C, int M, int vec,
                                    hipStream_t st) {
    const int64_t cw = 64 * vec;
    const int ts = shift_bwd_ts(vec);
    const int64_t ntcb = (T + kShiftBwdWaves * ts - 1) / (kShiftBwdWaves * ts);
    const int64_t nblk = B * ntcb;
    const dim3 grid((unsigned)(nblk * ((C + cw - 1) / cw)));
    if (vec == 2) launch_bwd<2, shift_bwd_ts(2)>(A, grid, B, T, C, M, st);
    else launch_bwd<1, shift_bwd_ts(1)>(A, grid, B, T, C, M, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(token_shift_mu_kernel, dim3((unsigned)(M * ((C + 63) / 64))), dim3(64 * kMuWaves), 0, st, A,
                       nblk, C, M);
    return hipGetLastError();
}

}  // namespace linrec

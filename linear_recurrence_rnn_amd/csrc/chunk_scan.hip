// chunk_scan.hip -- the scan kernel (scan_kernel.hpp) instantiated for the WKV-4 forward,
// the real and complex scans and their adjoints, and the small helper kernels of those
// entry points (fills, copies, the two-stage glambda sum of the complex adjoint).
#include "scan_kernel.hpp"

namespace linrec {

namespace {

using scan_kernel::dispatch;
using scan_kernel::dispatch_shape;

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.f;
}

// glam, first stage: block (group, k, b) adds slabs [k kPartBlock, (k+1) kPartBlock) of batch
// row b for its 64 channels, so that many rows of short sequences still fill the chip.  The
// association is fixed: slab s goes to accumulator s mod 8 (8 loads in flight at a time, not
// one) and the 8 accumulators are added in order.
__global__ __launch_bounds__(64) void part_sum_kernel(ScanGeom g) {
    const int64_t grp = blockIdx.x, k = blockIdx.y;
    const int lane = threadIdx.x;
    const int64_t c = grp * 64 + lane;
    if (c >= g.C) return;
    const int64_t nk = gridDim.y;
    const int64_t s0 = k * kPartBlock, s1 = min(g.nslab, s0 + kPartBlock);
    for (int64_t b = blockIdx.z; b < g.B; b += gridDim.z) {
        const double* p = g.part + 2 * (((b * g.ngrp + grp) * g.nslab) * 64 + lane);
        double ar[8], ai[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) ar[i] = ai[i] = 0.0;
        int64_t s = s0;
        for (; s + 8 <= s1; s += 8) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                ar[i] += p[2 * (s + i) * 64];
                ai[i] += p[2 * (s + i) * 64 + 1];
            }
        }
        for (int i = 0; s < s1; ++s, ++i) {
            ar[i] += p[2 * s * 64];
            ai[i] += p[2 * s * 64 + 1];
        }
        double re = 0.0, im = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            re += ar[i];
            im += ai[i];
        }
        g.part2[2 * ((b * nk + k) * g.C + c)] = re;
        g.part2[2 * ((b * nk + k) * g.C + c) + 1] = im;
    }
}

// glam, second stage: the first-stage sums of a channel (batch rows in ascending order,
// slab blocks within a row in order; entry e to accumulator e mod 8, added in order), as
// complex64 (or the real part alone as float32).
__global__ __launch_bounds__(256) void part_final_kernel(ScanGeom g, int64_t nk, float* __restrict__ glam,
                                                         bool complex_out) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= g.C) return;
    const int64_t n = g.B * nk;
    double ar[8], ai[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ar[i] = ai[i] = 0.0;
    int64_t e = 0;
    for (; e + 8 <= n; e += 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            ar[i] += g.part2[2 * ((e + i) * g.C + c)];
            ai[i] += g.part2[2 * ((e + i) * g.C + c) + 1];
        }
    }
    for (int i = 0; e < n; ++e, ++i) {
        ar[i] += g.part2[2 * (e * g.C + c)];
        ai[i] += g.part2[2 * (e * g.C + c) + 1];
    }
    double re = 0.0, im = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        re += ar[i];
        im += ai[i];
    }
    if (complex_out) {
        glam[2 * c] = (float)re;
        glam[2 * c + 1] = (float)im;
    } else {
        glam[c] = (float)re;
    }
}

}  // namespace

bool scan_shape_supported(int kind, int vec, int nw, int L) {
    const int vmax = is_bwd_kind(kind) ? 1 : ((kind == kKindWkv || kind == kKindReal) ? 4 : 2);
    const bool vec_ok = vec == vmax || (vec == 2 && vmax >= 2) || vec == 1;
    return vec_ok && ((nw == 4 && L == 16) || (nw == 8 && L == 8) || (nw == 8 && L == 16) ||
                      (kind != kKindWkv && vec == 1 && nw == 8 && L == 32));
}

// A carried state or a gate takes the extended instance; the plain call compiles none of it.
hipError_t run_wkv_forward(const WkvArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st) {
    if (A.r || A.s_in || A.s_out) return dispatch<WkvExtOp, 4>(A, g, p, st);
    return dispatch<WkvOp, 4>(A, g, p, st);
}
hipError_t run_scan_real(const RealArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st) {
    return dispatch<RealOp, 4>(A, g, p, st);
}
hipError_t run_scan_complex(const CplxArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st) {
    return dispatch<CplxOp, 2>(A, g, p, st);
}
// The adjoints keep one channel per lane (their steps also hold x_{t-1}).
hipError_t run_scan_real_backward(const RealBwdArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st) {
    if (p.vec != 1) return hipErrorInvalidValue;
    return dispatch_shape<RealBwdOp, 1>(A, g, p, st);
}
hipError_t run_scan_complex_backward(const CplxBwdArgs& A, float* glam, const ScanGeom& g, const ScanPlan& p,
                                     hipStream_t st) {
    if (p.vec != 1) return hipErrorInvalidValue;
    const hipError_t e = dispatch_shape<CplxBwdOp, 1>(A, g, p, st);
    return e != hipSuccess ? e : run_part_sums(g, glam, true, st);
}

hipError_t run_part_sums(const ScanGeom& g, float* glam, bool complex_out, hipStream_t st) {
    const int64_t nk = (g.nslab + kPartBlock - 1) / kPartBlock;
    const unsigned nb = (unsigned)(g.B < 65535 ? g.B : 65535);
    hipLaunchKernelGGL(part_sum_kernel, dim3((unsigned)g.ngrp, (unsigned)nk, nb), dim3(64), 0, st, g);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(part_final_kernel, dim3((unsigned)((g.C + 255) / 256)), dim3(256), 0, st, g, nk, glam,
                       complex_out);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void copy_kernel(float* __restrict__ d, const float* __restrict__ s, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        d[i] = s[i];
}

hipError_t run_copy(float* dst, const float* src, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, st, dst, src, n);
    return hipGetLastError();
}

hipError_t run_fill_zero(float* p, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

size_t agg_bytes(int kind) {
    switch (kind) {
        case kKindWkv: return sizeof(WkvOp::Agg);
        case kKindReal:
        case kKindRealBwd:
        case kKindMinGru:
        case kKindMinLstm:
        case kKindMinGruBwd:
        case kKindMinLstmBwd: return sizeof(RealOp::Agg);
        case kKindRealDecay:
        case kKindRealDecayBwd: return sizeof(RealDecayOp::Agg);
        default: return sizeof(CplxOp::Agg);
    }
}

}  // namespace linrec

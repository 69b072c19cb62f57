// chunk_scan.hip -- the scan kernel (scan_kernel.hpp) instantiated for the WKV-4 forward,
// the real and complex scans and their adjoints, and the small helper kernels of those
// entry points (fills, copies, the glambda sums of the adjoints: part_reduce.hpp).
#include "part_reduce.hpp"
#include "scan_kernel.hpp"

namespace linrec {

namespace {

using scan_kernel::dispatch;
using scan_kernel::dispatch_shape;

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.f;
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
    const unsigned nb = (unsigned)(g.B < 65535 ? g.B : 65535);
    hipLaunchKernelGGL(part_sum_kernel, dim3((unsigned)g.ngrp, (unsigned)g.nk, nb), dim3(64 * kPartWaves), 0, st, g);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(part_final_kernel, dim3((unsigned)g.ngrp), dim3(64 * kPartWaves), 0, st, g, glam, complex_out);
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

hipError_t clear_flags_if_capturing(uint64_t* flags, int64_t n, hipStream_t st) {
    if (!flags || n <= 0) return hipSuccess;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    const hipError_t e = hipStreamIsCapturing(st, &cs);
    if (e != hipSuccess) return e;
    if (cs != hipStreamCaptureStatusActive) return hipSuccess;
    return run_fill_zero(reinterpret_cast<float*>(flags), 2 * n, st);
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

// scan_variants.hip -- the scan kernel (scan_kernel.hpp) instantiated for the gated variants:
// minGRU and minLSTM from gate pre-activations, the real scan with one decay per channel,
// and the LRU with normalised input (operators in scan_ops.hpp).  A separate source so the
// instantiations compile beside those of chunk_scan.hip.
#include "scan_kernel.hpp"

namespace linrec {

hipError_t run_scan_mingru(const MinGruArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st) {
    return scan_kernel::dispatch<MinGruOp, 2>(A, g, p, st);
}
hipError_t run_scan_minlstm(const MinLstmArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st) {
    return scan_kernel::dispatch<MinLstmOp, 2>(A, g, p, st);
}
hipError_t run_scan_real_decay(const RealDecayArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st) {
    return scan_kernel::dispatch<RealDecayOp, 2>(A, g, p, st);
}
hipError_t run_scan_complex_normalized(const CplxArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st) {
    return scan_kernel::dispatch<CplxNormOp, 2>(A, g, p, st);
}

// The adjoints keep one channel per lane (their steps also hold x_{t-1} and the gates).
hipError_t run_scan_mingru_backward(const MinGruBwdArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st) {
    if (p.vec != 1) return hipErrorInvalidValue;
    return scan_kernel::dispatch_shape<MinGruBwdOp, 1>(A, g, p, st);
}
hipError_t run_scan_minlstm_backward(const MinLstmBwdArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st) {
    if (p.vec != 1) return hipErrorInvalidValue;
    return scan_kernel::dispatch_shape<MinLstmBwdOp, 1>(A, g, p, st);
}
hipError_t run_scan_real_decay_backward(const RealDecayBwdArgs& A, float* glam, const ScanGeom& g, const ScanPlan& p,
                                        hipStream_t st) {
    if (p.vec != 1) return hipErrorInvalidValue;
    const hipError_t e = scan_kernel::dispatch_shape<RealDecayBwdOp, 1>(A, g, p, st);
    return e != hipSuccess ? e : run_part_sums(g, glam, false, st);
}
hipError_t run_scan_complex_normalized_backward(const CplxBwdArgs& A, float* glam, const ScanGeom& g,
                                                const ScanPlan& p, hipStream_t st) {
    if (p.vec != 1 || !A.u) return hipErrorInvalidValue;
    const hipError_t e = scan_kernel::dispatch_shape<CplxNormBwdOp, 1>(A, g, p, st);
    return e != hipSuccess ? e : run_part_sums(g, glam, true, st);
}

}  // namespace linrec

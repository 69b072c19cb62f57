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

}  // namespace linrec

// wkv_decode.hip -- one token of the WKV-4 operator in its recurrent form (token-by-token
// decoding): the output and the state update of eq. (14) on the RWKV-LLM page ("Time-mixing
// block") for a single time step, gated by sigma(r) as in eq. (15).
//
// From the carried past sums A, B (state (a, b, p), A = a e^p, B = b e^p):
//   y  = sigma(r) (A + e^{u+k} v) / (B + e^{u+k})
//   A' = e^{-w} A + e^{k} v,   B' = e^{-w} B + e^{k}
// evaluated as the per-step update of the forward (integer base-2 exponents, running
// maximum; see wkv_math.hpp), so a sequence decoded token by token follows the same
// arithmetic as the chunked forward's exact path.
//
// One lane per (batch row, channel); the work is a few hundred bytes per batch row and
// channel-contiguous, so it is bound by launch latency rather than by any unit of the chip.
#include "wkv_decode.hpp"
#include "device_common.hpp"
#include "wkv_math.hpp"

namespace linrec {

namespace {

__global__ __launch_bounds__(256) void wkv_decode_step_kernel(WkvStepArgs A, int64_t B, int64_t C) {
    const int64_t n = B * C;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t c = i % C;
        const float om = fminf(A.w[c] * kLog2e, kMaxOm), mu = A.u[c] * kLog2e;
        const float kk = A.k[i] * kLog2e, vv = A.v[i];
        float* s = A.state + 3 * i;
        const Base2State x = state_from_natural(s[0], s[1], s[2]);
        const float m = mag(x.p, x.b);
        // Output: both terms at the exponent q of the larger one.
        const float q = ceilf(fmaxf(m, kk + mu));
        const float e1 = fast_exp2(x.p - q), e2 = fast_exp2((kk - q) + mu);
        float y = fmaf(x.a, e1, vv * e2) * __builtin_amdgcn_rcpf(fmaf(x.b, e1, e2));
        if (A.r) y *= __builtin_amdgcn_rcpf(1.f + fast_exp2(-A.r[i] * kLog2e));
        // Update: decay the past by e^{-w}, add this token.
        const float q2 = ceilf(fmaxf(m - om, kk));
        const float f1 = fast_exp2((x.p - q2) - om), f2 = fast_exp2(kk - q2);
        const Base2State nx{fmaf(x.a, f1, vv * f2), fmaf(x.b, f1, f2), q2};
        float oa, ob, op;
        state_to_natural(nx, oa, ob, op);
        A.y[i] = y;
        s[0] = oa;
        s[1] = ob;
        s[2] = op;
    }
}

}  // namespace

hipError_t run_wkv_decode_step(const WkvStepArgs& A, int64_t B, int64_t C, hipStream_t st) {
    const int64_t n = B * C;
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(wkv_decode_step_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, st,
                       A, B, C);
    return hipGetLastError();
}

}  // namespace linrec

// token_shift.hpp -- host-visible interface of the token-shift kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace linrec {

struct TokenShiftArgs {
    const float* x;       // (B,T,C)
    const float* x_prev;  // (B,C) token before x[:,0], or null (zero)
    const float* mu;      // (M,C)
    float* out;           // (M,B,T,C)
};

struct TokenShiftBwdArgs {
    const float* x;       // (B,T,C)
    const float* x_prev;  // (B,C) or null
    const float* mu;      // (M,C)
    const float* g;       // (M,B,T,C) dL/dout
    float* gx;            // (B,T,C)
    float* gmu;           // (M,C)
    float* gx_prev;       // (B,C) or null
    double* part;         // workspace: per-block dL/dmu sums
};

constexpr int kShiftMaxM = 4;  // mixes per call

// vec: channels per lane (1, 2 or 4; 4 and 2 need C and the pointers to allow them).
hipError_t run_token_shift(const TokenShiftArgs& A, int64_t B, int64_t T, int64_t C, int M, int vec,
                           hipStream_t st);
size_t token_shift_backward_ws_bytes(int64_t B, int64_t T, int64_t C, int M, int vec);
hipError_t run_token_shift_backward(const TokenShiftBwdArgs& A, int64_t B, int64_t T, int64_t C, int M, int vec,
                                    hipStream_t st);

}  // namespace linrec

// wkv_decode.hpp -- host-visible interface of the one-token WKV-4 step (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace linrec {

struct WkvStepArgs {
    const float* w;  // (C)
    const float* u;  // (C)
    const float* k;  // (B,C) this token
    const float* v;  // (B,C)
    const float* r;  // (B,C) receptance, or null (no gate)
    float* state;    // (B,C,3) (a, b, p), read and then overwritten in place
    float* y;        // (B,C)
};

hipError_t run_wkv_decode_step(const WkvStepArgs& A, int64_t B, int64_t C, hipStream_t st);

}  // namespace linrec

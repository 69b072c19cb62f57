// wkv_backward.hpp -- host-visible interface of the WKV-4 backward kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace linrec {

struct WkvBwdArgs {
    const float* w;   // (C)
    const float* u;   // (C)
    const float* k;   // (B,T,C)
    const float* v;   // (B,T,C)
    const float* gy;  // (B,T,C)
    float* gw;        // (C)
    float* gu;        // (C)
    float* gk;        // (B,T,C)
    float* gv;        // (B,T,C)
};

struct BwdPlan {
    int vec;         // channels per lane: 2 or 1
    int64_t ntiles;  // tiles of the time axis
    size_t ckpt_bytes;
    size_t ws_bytes;
};

BwdPlan wkv_backward_plan(int64_t B, int64_t T, int64_t C);
hipError_t run_wkv_backward(const WkvBwdArgs& A, int64_t B, int64_t T, int64_t C, const BwdPlan& p,
                            void* ws, hipStream_t st);
// Writes zeros to gw and gu (C floats each): the sums over an empty batch or sequence.
hipError_t run_zero_wu(float* gw, float* gu, int64_t C, hipStream_t st);

}  // namespace linrec

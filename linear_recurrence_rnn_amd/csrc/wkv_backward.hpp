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
    const float* r;   // (B,T,C) receptance of the gated output sigma(r) wkv, or null
    float* gr;        // (B,T,C) dL/dr when r is given
    const float* s_in;    // (B,C,3) carried state (a, b, p) before the first token, or null
    const float* s_out;   // (B,C,3) the forward's state after the last token (its p), or null
    const float* gs_out;  // (B,C,2) dL/d(a', b') of s_out (p' fixed), or null
    float* gs_in;         // (B,C,2) dL/d(a, b) of s_in (its p fixed), or null
};

// Launch geometry of the backward.  The gradient kernel cuts each sequence into slabs of nw
// chunks of L steps of one channel group (64 lanes x vec channels) and visits them in
// reverse time order (workgroups numbered chain-major); the state kernel writes the forward
// sums at every slab end, looking back over items of several slabs in time order.
struct BwdGeom {
    int64_t B, T, C;
    int64_t ngrp;   // channel groups per batch row
    int64_t nslab;  // slabs per sequence
    int spin;       // polls of a predecessor's flag before recomputing its aggregate
    uint64_t tag_f, tag_r;  // per-call tags of the two kernels' flags (never 0)
    uint64_t* flags_c;      // forward (coarse) chain of the state kernel: flags per item
    void* agg_c;            // (B*ngrp*items, 64*vec) item aggregates
    void* incl_c;           // (B*ngrp*items, 64*vec) item inclusive prefixes
    void* incl_f;           // (B*ngrp*nslab, 64*vec) forward sums at the end of every slab
    uint64_t* flags_r;      // reverse-chain flags, records indexed by chain position
    void* agg_r;
    void* incl_r;
    double* part;           // (B, C, 2) dL/dw, dL/du of each batch row
    int exact_only;         // 1: the gradient kernel never takes its frame fast path (tests)
    int from_ckpt;          // 1: incl_f holds a checkpointing forward's sums; no state kernel
};

struct BwdPlan {
    int vec;        // channels per lane (1)
    int nw;         // waves per workgroup (chunks per slab)
    int L;          // steps per chunk
    int64_t nslab;  // slabs per sequence
    size_t ws_bytes;
};

// Plan (nw, L from the defaults or the overrides, when a kernel of that shape exists).
BwdPlan wkv_backward_plan(int vec, int64_t B, int64_t T, int64_t C, int nw_override, int L_override);
// Workspace layout of a plan: fills the pointers of g from ws.
void wkv_backward_layout(const BwdPlan& p, int64_t B, int64_t C, void* ws, BwdGeom& g);
bool bwd_shape_supported(int vec, int nw, int L);
hipError_t run_wkv_backward(const WkvBwdArgs& A, const BwdGeom& g, const BwdPlan& p, hipStream_t st);
// Writes zeros to gw and gu (C floats each): the sums over an empty batch or sequence.
hipError_t run_zero_wu(float* gw, float* gu, int64_t C, hipStream_t st);
// No tokens: the state passes through, so gs_in = gs_out e^{p_in - p_out} (zero without gs_out).
hipError_t run_state_grad_passthrough(const WkvBwdArgs& A, int64_t B, int64_t C, hipStream_t st);

// The checkpointing forward (wkv_ckpt.hip): y as wkv4_forward, and the forward sums at the end
// of every slab of the default backward plan written to ckpt (the layout of incl_f).
// Checkpoint bytes, forward workspace bytes, and the launch (ws holds flags and aggregates).
size_t wkv_ckpt_bytes(int64_t B, int64_t T, int64_t C);
size_t wkv_ckpt_forward_ws_bytes(int64_t B, int64_t T, int64_t C);
struct WkvArgs;
// The backward from such checkpoints: workspace bytes (dL/dw, dL/du rows and the reverse
// look-back only) and the layout, with incl_f = ckpt and the state kernel skipped.
size_t wkv_backward_ckpt_ws_bytes(int64_t B, int64_t T, int64_t C);
void wkv_backward_layout_ckpt(const BwdPlan& p, int64_t B, int64_t C, void* ws, const void* ckpt, BwdGeom& g);
hipError_t run_wkv_forward_ckpt(const WkvArgs& A, int64_t B, int64_t T, int64_t C, void* ckpt, void* ws,
                                uint64_t tag, int spin, bool sep, hipStream_t st);

}  // namespace linrec

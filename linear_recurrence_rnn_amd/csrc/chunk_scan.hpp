// chunk_scan.hpp -- host-visible interface of the forward scan kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace linrec {

enum { kKindWkv = 0, kKindReal = 1, kKindComplex = 2 };

// Operands of each recurrence (device pointers, (B,T,C) row-major, C fastest).
struct WkvArgs {
    const float* w;  // (C)
    const float* u;  // (C)
    const float* k;  // (B,T,C)
    const float* v;  // (B,T,C)
    float* y;        // (B,T,C)
    int exact_only;  // 1: always take the exact per-step path (used by tests)
};
struct RealArgs {
    const float* a;   // (B,T,C)
    const float* b;   // (B,T,C)
    const float* x0;  // (B,C) or null
    float* x;         // (B,T,C)
};
struct CplxArgs {
    const float* lam;  // (C) complex64
    const float* u;    // (B,T,C) complex64
    const float* x0;   // (B,C) complex64 or null
    float* x;          // (B,T,C) complex64
};

// Launch geometry.  A workgroup of nw waves owns one time slab (nw chunks of L steps) of
// one channel group (64 lanes x vec channels); workgroups are numbered slab-major, so a
// slab's predecessors always have smaller block indices.
struct ScanGeom {
    int64_t B, T, C;
    int64_t ngrp;       // channel groups per batch row
    int64_t nslab;      // slabs per sequence
    uint64_t tag;       // per-call tag of the look-back flags (never 0)
    int spin;           // polls of a predecessor's flag before recomputing its aggregate
    uint64_t* flags;    // (B*ngrp*nslab) publication flags
    void* rec_agg;      // (B*ngrp*nslab, 64*vec) slab aggregates
    void* rec_incl;     // (B*ngrp*nslab, 64*vec) inclusive prefixes
};

struct ScanPlan {
    int vec;        // channels per lane (4, or 2 for complex; 1 for any C or alignment)
    int nw;         // waves per workgroup (chunks per slab)
    int L;          // steps per chunk
    int64_t nslab;  // slabs per sequence
    size_t ws_bytes;
};

hipError_t run_wkv_forward(const WkvArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st);
hipError_t run_scan_real(const RealArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st);
hipError_t run_scan_complex(const CplxArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st);
size_t agg_bytes(int kind);
// Launch shapes that have kernels: (vec, nw, L) per kind.
bool scan_shape_supported(int kind, int vec, int nw, int L);

}  // namespace linrec

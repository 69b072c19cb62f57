// chunk_scan.hpp -- host-visible interface of the chunked-scan kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace linrec {

// Steps per chunk held in registers by one workgroup row.
constexpr int kChunkLen = 16;
// Channels per workgroup (CL lanes x VEC channels per lane).
constexpr int kGroupChannels = 16;

enum { kModeFull = 0, kModeReduce = 1, kModeApply = 2 };
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

struct ScanGeom {
    int64_t B, T, C;
    int64_t ngrp;      // channel groups of kGroupChannels channels
    int64_t nslab;     // time slabs per sequence (1: one workgroup walks the whole sequence)
    int64_t slab_len;  // steps per slab, a multiple of the tile length
    int mode;          // kMode*
    void* ws_agg;      // (B, nslab, C) slab aggregates
    void* ws_carry;    // (B, nslab, C) slab carries
};

struct ScanPlan {
    int vec;       // channels per lane: 4 (2 for complex) or 1
    int rows;      // chunks per tile: 64 or 16
    int64_t nslab;
    int64_t slab_len;
    size_t ws_bytes;
};

hipError_t run_wkv_forward(const WkvArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st);
hipError_t run_scan_real(const RealArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st);
hipError_t run_scan_complex(const CplxArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st);
size_t agg_bytes(int kind);

}  // namespace linrec

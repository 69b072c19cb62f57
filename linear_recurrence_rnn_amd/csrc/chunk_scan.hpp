// chunk_scan.hpp -- host-visible interface of the forward scan kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace linrec {

enum { kKindWkv = 0, kKindReal = 1, kKindComplex = 2, kKindRealBwd = 3, kKindComplexBwd = 4,
       kKindMinGru = 5, kKindMinLstm = 6, kKindRealDecay = 7, kKindComplexNorm = 8,
       kKindMinGruBwd = 9, kKindMinLstmBwd = 10, kKindRealDecayBwd = 11, kKindComplexNormBwd = 12 };

// Kinds of the reverse-time adjoints (one channel per lane).
inline bool is_bwd_kind(int kind) {
    return kind == kKindRealBwd || kind == kKindComplexBwd || kind >= kKindMinGruBwd;
}
// Kinds whose adjoint sums a per-channel gradient over batch and time (glambda).
inline bool has_parts(int kind) {
    return kind == kKindComplexBwd || kind == kKindRealDecayBwd || kind == kKindComplexNormBwd;
}

// Operands of each recurrence (device pointers, (B,T,C) row-major, C fastest).
struct WkvArgs {
    const float* w;     // (C)
    const float* u;     // (C)
    const float* k;     // (B,T,C)
    const float* v;     // (B,T,C)
    float* y;           // (B,T,C)
    int exact_only;     // 1: always take the exact per-step path (used by tests)
    const float* r;     // (B,T,C) receptance, or null: y = sigma(r) wkv
    const float* s_in;  // (B,C,3) state (a, b, p) before the first token, or null (empty)
    float* s_out;       // (B,C,3) state after the last token, or null
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
// Gated variants of the real scan (coefficients formed from the gates in the kernel).
struct MinGruArgs {
    const float* kz;  // (B,T,C) gate pre-activation: z = sigmoid(kz)
    const float* h;   // (B,T,C) candidate h~
    const float* x0;  // (B,C) or null
    float* x;         // (B,T,C)
};
struct MinLstmArgs {
    const float* kf;  // (B,T,C) forget-gate pre-activation
    const float* ki;  // (B,T,C) input-gate pre-activation
    const float* h;   // (B,T,C) candidate h~
    const float* x0;  // (B,C) or null
    float* x;         // (B,T,C)
};
struct RealDecayArgs {
    const float* lam;  // (C) decay per channel
    const float* u;    // (B,T,C)
    const float* x0;   // (B,C) or null
    float* x;          // (B,T,C)
};
// Adjoints of the two linear scans (reverse time).
struct RealBwdArgs {
    const float* a;   // (B,T,C)
    const float* x0;  // (B,C) or null
    const float* x;   // (B,T,C) forward output
    const float* gx;  // (B,T,C) dL/dx
    float* ga;        // (B,T,C)
    float* gb;        // (B,T,C)
    float* gx0;       // (B,C) or null
};
struct CplxBwdArgs {
    const float* lam;  // (C) complex64
    const float* x0;   // (B,C) complex64 or null
    const float* x;    // (B,T,C) complex64 forward output
    const float* gx;   // (B,T,C) complex64 dL/dx
    float* gu;         // (B,T,C) complex64
    float* gx0;        // (B,C) complex64 or null
    const float* u;    // (B,T,C) complex64 input (normalised LRU only: dL/dgamma), else null
};
// Adjoints of the gated variants.
struct MinGruBwdArgs {
    const float* kz;  // (B,T,C)
    const float* h;   // (B,T,C)
    const float* x0;  // (B,C) or null
    const float* x;   // (B,T,C) forward output
    const float* gx;  // (B,T,C) dL/dx
    float* gkz;       // (B,T,C)
    float* gh;        // (B,T,C)
    float* gx0;       // (B,C) or null
};
struct MinLstmBwdArgs {
    const float* kf;  // (B,T,C)
    const float* ki;  // (B,T,C)
    const float* h;   // (B,T,C)
    const float* x0;  // (B,C) or null
    const float* x;   // (B,T,C) forward output
    const float* gx;  // (B,T,C) dL/dx
    float* gkf;       // (B,T,C)
    float* gki;       // (B,T,C)
    float* gh;        // (B,T,C)
    float* gx0;       // (B,C) or null
};
struct RealDecayBwdArgs {
    const float* lam;  // (C)
    const float* x0;   // (B,C) or null
    const float* x;    // (B,T,C) forward output
    const float* gx;   // (B,T,C) dL/dx
    float* gu;         // (B,T,C)
    float* gx0;        // (B,C) or null
};

// Addressing of a run of consecutive steps (a chunk, or a slab being recomputed): logical
// step j sits at byte offset soff(j) from the run's buffer base (its lowest row) and at
// time t(j) of the sequence.  Scans in time order have rstep = +row bytes, tdir = +1;
// scans in reverse time start from the run's last row.
struct Rows {
    unsigned s0;   // byte offset of logical step 0
    int rstep;     // bytes from one logical step to the next (negative in reverse time)
    int64_t t0;    // time of logical step 0
    int tdir;      // +1 or -1
    __device__ __forceinline__ unsigned soff(int j) const { return s0 + (unsigned)(j * rstep); }
    __device__ __forceinline__ int64_t t(int j) const { return t0 + (int64_t)j * tdir; }
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
    double* part;       // (B*ngrp*nslab, 64*vec, 2) per-slab sums of operators that have them
    double* part2;      // (B*nk, C, 2) their first-stage sums (see run_scan_complex_backward)
    int64_t nk;         // ceil(nslab / kPartBlock): first-stage blocks per row
};

struct ScanPlan {
    int vec;        // channels per lane (4, or 2 for complex; 1 for any C or alignment)
    int nw;         // chunks per slab (waves per workgroup, one more with sep)
    int L;          // steps per chunk
    bool sep;       // a coordinator wave of its own (one channel per lane only)
    int64_t nslab;  // slabs per sequence
    size_t ws_bytes;
};

hipError_t run_wkv_forward(const WkvArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st);
hipError_t run_scan_real(const RealArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st);
hipError_t run_scan_complex(const CplxArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st);
hipError_t run_scan_mingru(const MinGruArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st);
hipError_t run_scan_minlstm(const MinLstmArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st);
hipError_t run_scan_real_decay(const RealDecayArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st);
hipError_t run_scan_complex_normalized(const CplxArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st);
hipError_t run_scan_real_backward(const RealBwdArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st);
hipError_t run_scan_mingru_backward(const MinGruBwdArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st);
hipError_t run_scan_minlstm_backward(const MinLstmBwdArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st);
// Also sums the per-slab shares of dL/dlam into glam (C float32).
hipError_t run_scan_real_decay_backward(const RealDecayBwdArgs& A, float* glam, const ScanGeom& g, const ScanPlan& p,
                                        hipStream_t st);
// As run_scan_complex_backward, with A.u the input scaled by gamma.
hipError_t run_scan_complex_normalized_backward(const CplxBwdArgs& A, float* glam, const ScanGeom& g,
                                                const ScanPlan& p, hipStream_t st);
// Sums g.part (per-slab shares, pairs) over slabs and batch rows into glam: C complex64
// (`complex_out`) or C float32 (the first of each pair).
hipError_t run_part_sums(const ScanGeom& g, float* glam, bool complex_out, hipStream_t st);
// Also sums g.part into glam (C complex64): g.part2 holds B x ceil(nslab / kPartBlock) x C pairs.
hipError_t run_scan_complex_backward(const CplxBwdArgs& A, float* glam, const ScanGeom& g, const ScanPlan& p,
                                     hipStream_t st);
constexpr int kPartBlock = 64;  // slabs summed per first-stage block of the glam reduction
// Writes n zero floats (a fill kernel: the library records no memset).
hipError_t run_fill_zero(float* p, int64_t n, hipStream_t st);
// A call recorded into a HIP graph keeps its host-drawn tag on every replay, so the flags a
// replay publishes would meet the previous replay's.  While `st` is capturing, this records
// a fill kernel that zeroes the n flags first ("not published"); otherwise it does nothing.
hipError_t clear_flags_if_capturing(uint64_t* flags, int64_t n, hipStream_t st);
// dst[i] = src[i] for n floats (a copy kernel, for the same reason).
hipError_t run_copy(float* dst, const float* src, int64_t n, hipStream_t st);
size_t agg_bytes(int kind);
// Launch shapes that have kernels: (vec, nw, L) per kind.
bool scan_shape_supported(int kind, int vec, int nw, int L);

}  // namespace linrec

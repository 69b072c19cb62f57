// chunk_scan.hip -- single-pass, time-parallel evaluation of a first-order recurrence on gfx950.
//
// Layout.  A channel group is 64 lanes x VEC channels (1 KB of float32 per time step for
// VEC = 4), so every wave-wide load or store touches one contiguous row segment.  A
// workgroup of NW waves owns one slab of NW*L time steps of one group; wave w holds chunk w,
// steps [w*L, (w+1)*L) of the slab, in registers.  Every input element is read from HBM
// once and every output written once.
//
//   phase 1  each wave reduces its chunk to an aggregate (from the identity state);
//   phase 2  the NW chunk aggregates are scanned through LDS;
//   carry    wave 0 publishes the slab aggregate, then looks back over the earlier slabs
//            of the same group (decoupled look-back, 64 slabs per round trip, one per lane)
//            for the nearest published inclusive prefix, folds the aggregates after it in
//            time order (the association a chained scan would use: results do not depend
//            on timing), and publishes the slab's own inclusive prefix;
//   phase 3  each wave re-runs its chunk from its carry-in, straight from registers.
// The combine of two spans is associative, which is what lets a sequence be cut into
// chunks and slabs (the two-halves split of the LRU write-up, parallelisation section).
//
// Progress: workgroups are numbered slab-major, so a slab's predecessors have smaller block
// indices and are dispatched first.  A wait is bounded all the same: if a predecessor has
// not published after g.spin polls, the waiting wave recomputes that slab's aggregate from
// its inputs.  No wait depends on dispatch order or on the workspace contents; flags carry
// a per-call tag, so stale flags from earlier calls read as "not published".
#include "chunk_scan.hpp"
#include "scan_ops.hpp"

namespace linrec {

namespace {

constexpr uint64_t kStateAgg = 1;     // flag = tag * 4 + state
constexpr uint64_t kStateIncl = 2;

// Look-back records are written and read with device-scope relaxed atomics, which the
// hardware keeps coherent across the XCDs' L2 caches (write-through / coherent read), and
// a publication flag is stored only after all of the wave's record stores have completed
// (s_waitcnt).  This avoids agent-scope release/acquire fences, whose L2 writeback or
// invalidation serialises per XCD.
template <class T>
__device__ __forceinline__ void store_coherent(T* dst, const T& v) {
    static_assert(sizeof(T) % 4 == 0, "record must be whole dwords");
    uint32_t w[sizeof(T) / 4];
    __builtin_memcpy(w, &v, sizeof(T));
    uint32_t* d = reinterpret_cast<uint32_t*>(dst);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 4); ++i) __hip_atomic_store(d + i, w[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class T>
__device__ __forceinline__ T load_coherent(const T* src) {
    uint32_t w[sizeof(T) / 4];
    const uint32_t* s = reinterpret_cast<const uint32_t*>(src);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 4); ++i) w[i] = __hip_atomic_load(s + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    T v;
    __builtin_memcpy(&v, w, sizeof(T));
    return v;
}

// All of this wave's memory operations have completed (compiler and hardware ordering).
__device__ __forceinline__ void wait_memory() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wave-uniform copy of lane 0's 64-bit value (readfirstlane moves 32 bits).
__device__ __forceinline__ uint64_t first_lane_u64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t poll_flag(const uint64_t* f, uint64_t tag, int spin) {
    uint64_t v = 0;
    for (int it = 0; it < spin; ++it) {
        v = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((v >> 2) == tag) break;
        __builtin_amdgcn_s_sleep(2);
    }
    return v;
}

template <class Op, int VEC, int NW, int L>
__global__ __launch_bounds__(64 * NW) void lookback_scan_kernel(typename Op::Args A, ScanGeom g) {
    using Agg = typename Op::Agg;
    using In = typename Op::In;
    using Chan = typename Op::Chan;
    constexpr int CW = 64 * VEC;
    constexpr int SLAB = NW * L;
    constexpr int EF = Op::kFloats;
    __shared__ Agg sh[NW][CW];
    __shared__ Agg sh_carry[CW];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int64_t G = g.B * g.ngrp;
    const int64_t s = (int64_t)blockIdx.x / G;  // slab: slowest, so predecessors come first
    const int64_t gi = (int64_t)blockIdx.x - s * G;
    const int64_t b = gi / g.ngrp, grp = gi - b * g.ngrp;
    const int64_t c0 = grp * CW + (int64_t)lane * VEC;
    const bool active = c0 < g.C;  // C is a multiple of VEC
    const int64_t t_slab = s * SLAB;
    const int slab_n = (int)((g.T - t_slab) < SLAB ? (g.T - t_slab) : SLAB);
    const int n = active ? max(0, min(L, slab_n - w * L)) : 0;

    Chan ch[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) ch[e] = active ? Op::template chan<L>(A, c0 + e) : Chan{};

    const unsigned rowb = (unsigned)(g.C * EF * 4);           // bytes per time step
    const unsigned voff = (unsigned)(lane * VEC * EF * 4);    // this lane's bytes in the row
    const int64_t total = g.B * g.T * g.C;
    const int64_t base = (b * g.T + t_slab + (int64_t)w * L) * g.C + grp * CW;
    const typename Op::Res R = Op::res(A, base, (total - base) * EF * 4);
    In in[L][VEC];
    if (n == L) {
#pragma unroll
        for (int j = 0; j < L; ++j) Op::template load<VEC>(R, voff, j * rowb, in[j]);
    } else {
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) Op::template load<VEC>(R, voff, j * rowb, in[j]);
            else Op::template zero<VEC>(in[j]);
        }
    }

    // Phase 1: chunk aggregates.
    typename Op::Local loc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) sh[w][lane * VEC + e] = Op::template reduce<L, VEC>(ch[e], in, e, n, loc[e]);
    __syncthreads();

    // Phase 2: inclusive scan over the chunks of the slab.
    auto end_of = [&](int x) { return min((x + 1) * L, slab_n); };
#pragma unroll
    for (int d = 1; d < NW; d <<= 1) {
        Agg tmp[VEC];
        const bool has = w >= d;
        if (has) {
            const int n2 = end_of(w) - end_of(w - d);
#pragma unroll
            for (int e = 0; e < VEC; ++e) tmp[e] = Op::combine(ch[e], sh[w - d][lane * VEC + e], sh[w][lane * VEC + e], n2);
        }
        __syncthreads();
        if (has) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) sh[w][lane * VEC + e] = tmp[e];
        }
        __syncthreads();
    }

    // Carry into the slab (wave 0).
    if (w == 0) {
        const int64_t rec = gi * g.nslab + s;
        Agg* aggr = reinterpret_cast<Agg*>(g.rec_agg);
        Agg* incl = reinterpret_cast<Agg*>(g.rec_incl);
        const bool has_succ = s + 1 < g.nslab;
        if (has_succ) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) store_coherent(&aggr[rec * CW + lane * VEC + e], sh[NW - 1][lane * VEC + e]);
            wait_memory();
            if (lane == 0)
                __hip_atomic_store(g.flags + rec, g.tag * 4 + kStateAgg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // Look-back.  Phase A: lane i inspects slab hi-1-i, 64 predecessors per round trip,
        // until a round finds a published inclusive prefix (the nearest one, j0) or slab 0 is
        // passed (j0 = -1).  Lanes remember which slabs had published their aggregate.
        constexpr int kWin = 16;  // windows whose publication masks are kept
        uint64_t pub[kWin];
#pragma unroll
        for (int x = 0; x < kWin; ++x) pub[x] = 0;
        int64_t j0 = -1;
        int nwin = 0;
        for (int64_t hi = s; hi > 0; hi -= 64, ++nwin) {
            const int64_t j = hi - 1 - lane;
            const uint64_t f = (j >= 0) ? poll_flag(g.flags + gi * g.nslab + j, g.tag, g.spin) : 0;
            const uint64_t incl_mask = __ballot(j >= 0 && f == g.tag * 4 + kStateIncl);
            const uint64_t pub_mask = __ballot(j >= 0 && (f >> 2) == g.tag);
#pragma unroll
            for (int x = 0; x < kWin; ++x)
                if (x == nwin) pub[x] = pub_mask;
            if (incl_mask) {
                j0 = hi - 1 - (int64_t)(__ffsll((long long)incl_mask) - 1);
                break;
            }
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);  // record loads stay after the polls
        // Phase B: carry = INCL_j0 (or the initial state) folded left with A_{j0+1..s-1}: the
        // same association a strictly chained scan uses, so the result does not depend on
        // timing.  A slab whose aggregate was not published is recomputed from its inputs.
        Agg carry[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            if (j0 >= 0) carry[e] = load_coherent(&incl[(gi * g.nslab + j0) * CW + lane * VEC + e]);
            else carry[e] = active ? Op::init(A, b, c0 + e, g.C) : Op::identity();
        }
        // Records are fetched KB at a time (issued together, then folded in order) so the
        // fold costs one memory round trip per KB slabs.
        constexpr int KB = VEC >= 4 ? 2 : (VEC == 2 ? 4 : 8);
        for (int64_t j = j0 + 1; j < s; j += KB) {
            Agg xb[KB][VEC];
            bool pubb[KB];
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                const int64_t jj = j + k;
                pubb[k] = false;
                if (jj < s) {
                    const int64_t back = s - 1 - jj;  // lane index of slab jj in its window
                    const int x = (int)(back >> 6);
                    if (x < kWin) {
                        uint64_t m = 0;
#pragma unroll
                        for (int y = 0; y < kWin; ++y)
                            if (y == x) m = pub[y];
                        pubb[k] = (m >> (back & 63)) & 1;
                    } else {
                        uint64_t f = (lane == 0) ? poll_flag(g.flags + gi * g.nslab + jj, g.tag, g.spin) : 0;
                        pubb[k] = (first_lane_u64(f) >> 2) == g.tag;
                        __atomic_signal_fence(__ATOMIC_SEQ_CST);
                    }
                    if (pubb[k]) {
#pragma unroll
                        for (int e = 0; e < VEC; ++e)
                            xb[k][e] = load_coherent(&aggr[(gi * g.nslab + jj) * CW + lane * VEC + e]);
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                const int64_t jj = j + k;
                if (jj >= s) break;
                if (!pubb[k]) {
                    // Not published in time: recompute slab jj's aggregate from its inputs.
                    const int64_t bj = (b * g.T + jj * SLAB) * g.C + grp * CW;
                    const typename Op::Res Rj = Op::res(A, bj, (total - bj) * EF * 4);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) xb[k][e] = Op::identity();
                    if (active) {
                        for (int t = 0; t < SLAB; ++t) {
                            In xi[VEC];
                            Op::template load<VEC>(Rj, voff, t * rowb, xi);
#pragma unroll
                            for (int e = 0; e < VEC; ++e) xb[k][e] = Op::step(ch[e], xb[k][e], xi[e]);
                        }
                    }
                }
#pragma unroll
                for (int e = 0; e < VEC; ++e) carry[e] = Op::combine(ch[e], carry[e], xb[k][e], SLAB);
            }
        }
        if (has_succ) {
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                store_coherent(&incl[rec * CW + lane * VEC + e],
                               Op::combine(ch[e], carry[e], sh[NW - 1][lane * VEC + e], slab_n));
            wait_memory();
            if (lane == 0)
                __hip_atomic_store(g.flags + rec, g.tag * 4 + kStateIncl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) sh_carry[lane * VEC + e] = carry[e];
    }
    __syncthreads();

    // Phase 3: re-run my chunk from its carry-in.
    if (n > 0) {
        Agg cin[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            cin[e] = (w == 0) ? sh_carry[lane * VEC + e]
                              : Op::combine(ch[e], sh_carry[lane * VEC + e], sh[w - 1][lane * VEC + e], w * L);
        Op::template run<L, VEC>(R, ch, cin, in, loc, n, voff, rowb);
    }
}

template <class Op, int VEC, int NW, int L>
hipError_t launch(const typename Op::Args& A, const ScanGeom& g, hipStream_t st) {
    const int64_t nb = g.B * g.ngrp * g.nslab;
    hipLaunchKernelGGL((lookback_scan_kernel<Op, VEC, NW, L>), dim3((unsigned)nb), dim3(64 * NW), 0, st, A, g);
    return hipGetLastError();
}

// Kernels that exist: vec in {VMAX, 2, 1} x (nw, L) in {(4, 16), (8, 8), (8, 16)}.
template <class Op, int VEC>
hipError_t dispatch_shape(const typename Op::Args& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st) {
    if (p.nw == 4 && p.L == 16) return launch<Op, VEC, 4, 16>(A, g, st);
    if (p.nw == 8 && p.L == 8) return launch<Op, VEC, 8, 8>(A, g, st);
    if (p.nw == 8 && p.L == 16) return launch<Op, VEC, 8, 16>(A, g, st);
    return hipErrorInvalidValue;
}

template <class Op, int VMAX>
hipError_t dispatch(const typename Op::Args& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st) {
    if (p.vec == VMAX) return dispatch_shape<Op, VMAX>(A, g, p, st);
    if constexpr (VMAX > 2) {
        if (p.vec == 2) return dispatch_shape<Op, 2>(A, g, p, st);
    }
    if (p.vec == 1) return dispatch_shape<Op, 1>(A, g, p, st);
    return hipErrorInvalidValue;
}

}  // namespace

bool scan_shape_supported(int kind, int vec, int nw, int L) {
    const int vmax = kind == kKindComplex ? 2 : 4;
    const bool vec_ok = vec == vmax || vec == 2 || vec == 1;
    return vec_ok && ((nw == 4 && L == 16) || (nw == 8 && L == 8) || (nw == 8 && L == 16));
}

hipError_t run_wkv_forward(const WkvArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st) {
    return dispatch<WkvOp, 4>(A, g, p, st);
}
hipError_t run_scan_real(const RealArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st) {
    return dispatch<RealOp, 4>(A, g, p, st);
}
hipError_t run_scan_complex(const CplxArgs& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st) {
    return dispatch<CplxOp, 2>(A, g, p, st);
}

size_t agg_bytes(int kind) {
    switch (kind) {
        case kKindWkv: return sizeof(WkvOp::Agg);
        case kKindReal: return sizeof(RealOp::Agg);
        default: return sizeof(CplxOp::Agg);
    }
}

}  // namespace linrec

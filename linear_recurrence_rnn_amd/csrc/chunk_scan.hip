// chunk_scan.hip -- chunked, time-parallel evaluation of a first-order recurrence on gfx950.
//
// A workgroup owns a group of CW = CL*VEC consecutive channels of one batch row and walks
// a range of time steps in tiles of NR*L steps.  Inside a tile, row r of the workgroup
// (CL lanes, VEC channels per lane, channel-contiguous vector loads) holds chunk r, the L
// steps [r*L, (r+1)*L), in registers:
//   phase 1  each row reduces its chunk to an aggregate (from the identity state);
//   phase 2  the NR aggregates are scanned through LDS (Hillis-Steele, log2(NR) rounds);
//   phase 3  each row re-runs its chunk from its carry-in, straight from registers, and
//            stores the outputs.
// Every input element is read from HBM once and every output written once.
//
// When B*ceil(C/CW) workgroups would not fill the chip, the time axis is also cut into
// nslab slabs: a reduce pass writes each slab's aggregate to the workspace, a small
// kernel scans the slab aggregates of every channel into carries, and an apply pass
// re-runs each slab from its carry.  This costs one extra read of the inputs.
#include "chunk_scan.hpp"
#include "scan_ops.hpp"

namespace linrec {

template <class Op, int VEC, int CL, int NR, int L>
__global__ __launch_bounds__(CL * NR) void chunk_scan_kernel(typename Op::Args A, ScanGeom g) {
    using Agg = typename Op::Agg;
    using In = typename Op::In;
    using Chan = typename Op::Chan;
    constexpr int CW = CL * VEC;
    constexpr int TILE = NR * L;
    __shared__ Agg sh[NR][CW];

    const int tid = threadIdx.x;
    const int r = tid / CL;
    const int cl = tid - r * CL;
    const int64_t lb = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t grp = lb % g.ngrp;
    const int64_t rest = lb / g.ngrp;
    const int64_t s = rest % g.nslab;
    const int64_t b = rest / g.nslab;
    const int64_t c0 = grp * CW + (int64_t)cl * VEC;
    const bool active = c0 < g.C;  // C is a multiple of VEC
    const int64_t t_lo = s * g.slab_len;
    const int64_t t_hi = (t_lo + g.slab_len < g.T) ? t_lo + g.slab_len : g.T;

    Chan ch[VEC];
    Agg carry[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        ch[e] = active ? Op::template chan<L>(A, c0 + e) : Chan{};
        if (!active || g.mode == kModeReduce) {
            carry[e] = Op::identity();
        } else if (g.mode == kModeFull) {
            carry[e] = Op::init(A, b, c0 + e, g.C);
        } else {
            carry[e] = reinterpret_cast<const Agg*>(g.ws_carry)[(b * g.nslab + s) * g.C + c0 + e];
        }
    }

    for (int64_t t0 = t_lo; t0 < t_hi; t0 += TILE) {
        const int tt = (int)((t_hi - t0) < TILE ? (t_hi - t0) : TILE);  // steps in this tile
        const int n = max(0, min(L, tt - r * L));                          // steps in my chunk
        const int64_t off = (b * g.T + t0 + (int64_t)r * L) * g.C + c0;
        In in[L][VEC];
        if (active && n == L) {
#pragma unroll
            for (int j = 0; j < L; ++j) Op::template load<VEC>(A, off + (int64_t)j * g.C, in[j]);
        } else {
#pragma unroll
            for (int j = 0; j < L; ++j) {
                if (active && j < n) Op::template load<VEC>(A, off + (int64_t)j * g.C, in[j]);
                else Op::template zero<VEC>(in[j]);
            }
        }

        // Phase 1: chunk aggregates.
        typename Op::Local loc[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            sh[r][cl * VEC + e] = Op::template reduce<L, VEC>(ch[e], in, e, active ? n : 0, loc[e]);
        __syncthreads();

        // Phase 2: inclusive scan of the NR aggregates.  end(x) = steps from the tile
        // start through chunk x.
        auto end_of = [&](int x) { return min((x + 1) * L, tt); };
#pragma unroll
        for (int d = 1; d < NR; d <<= 1) {
            Agg tmp[VEC];
            const bool has = r >= d;
            if (has) {
                const int n2 = end_of(r) - end_of(r - d);
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    tmp[e] = Op::combine(ch[e], sh[r - d][cl * VEC + e], sh[r][cl * VEC + e], n2);
            }
            __syncthreads();
            if (has) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) sh[r][cl * VEC + e] = tmp[e];
            }
            __syncthreads();
        }

        // Phase 3: re-run my chunk from its carry-in.
        if (g.mode != kModeReduce && active && n > 0) {
            Agg cin[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                cin[e] = (r == 0) ? carry[e]
                                  : Op::combine(ch[e], carry[e], sh[r - 1][cl * VEC + e], end_of(r - 1));
            Op::template run<L, VEC>(A, ch, cin, in, loc, n, off, g.C);
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) carry[e] = Op::combine(ch[e], carry[e], sh[NR - 1][cl * VEC + e], tt);
        __syncthreads();
    }

    if (g.mode == kModeReduce && r == 0 && active) {
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            reinterpret_cast<Agg*>(g.ws_agg)[(b * g.nslab + s) * g.C + c0 + e] = carry[e];
    }
}

// Exclusive scan of the slab aggregates of one (batch, channel) into slab carries.
template <class Op, int L>
__global__ __launch_bounds__(256) void slab_carry_kernel(typename Op::Args A, ScanGeom g) {
    using Agg = typename Op::Agg;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= g.B * g.C) return;
    const int64_t b = i / g.C, c = i - b * g.C;
    const auto ch = Op::template chan<L>(A, c);
    Agg cur = Op::init(A, b, c, g.C);
    const Agg* agg = reinterpret_cast<const Agg*>(g.ws_agg);
    Agg* car = reinterpret_cast<Agg*>(g.ws_carry);
    for (int64_t s = 0; s < g.nslab; ++s) {
        const int64_t idx = (b * g.nslab + s) * g.C + c;
        car[idx] = cur;
        const int64_t rem = g.T - s * g.slab_len;
        cur = Op::combine(ch, cur, agg[idx], rem < g.slab_len ? rem : g.slab_len);
    }
}

template <class Op, int VEC, int NR>
static hipError_t launch(const typename Op::Args& A, ScanGeom g, hipStream_t st) {
    constexpr int L = kChunkLen;
    constexpr int CL = kGroupChannels / VEC;
    const int64_t nb = g.B * g.nslab * g.ngrp;
    if (g.nslab == 1) {
        g.mode = kModeFull;
        hipLaunchKernelGGL((chunk_scan_kernel<Op, VEC, CL, NR, L>), dim3((unsigned)nb), dim3(CL * NR),
                           0, st, A, g);
        return hipGetLastError();
    }
    g.mode = kModeReduce;
    hipLaunchKernelGGL((chunk_scan_kernel<Op, VEC, CL, NR, L>), dim3((unsigned)nb), dim3(CL * NR), 0,
                       st, A, g);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t nthreads = g.B * g.C;
    hipLaunchKernelGGL((slab_carry_kernel<Op, L>), dim3((unsigned)((nthreads + 255) / 256)), dim3(256),
                       0, st, A, g);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    g.mode = kModeApply;
    hipLaunchKernelGGL((chunk_scan_kernel<Op, VEC, CL, NR, L>), dim3((unsigned)nb), dim3(CL * NR), 0,
                       st, A, g);
    return hipGetLastError();
}

template <class Op, int VMAX>
static hipError_t dispatch(const typename Op::Args& A, const ScanGeom& g, const ScanPlan& p,
                           hipStream_t st) {
    if (p.vec == VMAX) {
        return p.rows == 64 ? launch<Op, VMAX, 64>(A, g, st) : launch<Op, VMAX, 16>(A, g, st);
    }
    return p.rows == 64 ? launch<Op, 1, 64>(A, g, st) : launch<Op, 1, 16>(A, g, st);
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

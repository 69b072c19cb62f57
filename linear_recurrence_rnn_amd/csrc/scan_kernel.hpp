// scan_kernel.hpp -- single-pass, time-parallel evaluation of a first-order recurrence on gfx950.
//
// Layout.  A channel group is 64 lanes x VEC channels (1 KB of float32 per time step for
// VEC = 4), so every wave-wide load or store touches one contiguous row segment.  A
// workgroup owns one slab of NW*L time steps of one group: wave w (of NW) holds chunk w,
// steps [w*L, (w+1)*L) of the slab, in registers.
// Every input element is read from HBM once and every output written once.
//
//   compute   each wave reduces its chunk to an aggregate (from the identity state);
//   carry     wave 0, its chunk parked in LDS, coordinates: it folds the chunk aggregates
//             into the slab aggregate, publishes it, looks back over the earlier slabs of
//             the same group (decoupled look-back, 64 slabs per round trip, one per lane) for
//             the nearest published inclusive prefix and folds the aggregates after it in
//             time order (the association a chained scan would use: results do not depend on
//             timing), and publishes the slab's own inclusive prefix;
//   re-run    each wave combines the slab's carry with the chunks before its own (prepared
//             by the coordinator) and re-runs its chunk straight from registers.
// In a chain short enough that all predecessors' records fit one batch (at most 1 + KB slabs)
// no inclusive prefix is published: every slab publishes its aggregate and folds all its
// predecessors' aggregates (look_back_short), one memory round trip instead of two.
// The waves meet at two barriers only.  Parking wave 0's chunk keeps the look-back's
// registers from adding to the chunk's, and having no wave without a chunk lets 3
// workgroups of 8 waves share a CU (the CU holds about 24 of these waves).  The combine of
// two spans is associative, which is what lets a sequence be cut into chunks and slabs (the
// two-halves split of the LRU write-up, parallelisation section).
//
// Progress: workgroups are numbered slab-major (a 3-D grid (groups, rows, slabs), or a flat
// one of the same order), so a slab's predecessors have smaller block indices and are
// dispatched first.  A wait is bounded all the same: if a predecessor has
// not published after g.spin polls, the waiting wave recomputes that slab's aggregate from
// its inputs.  No wait depends on dispatch order or on the workspace contents; flags carry
// a per-call tag, so stale flags from earlier calls read as "not published".
#pragma once

#include <cstdlib>
#include <type_traits>

#include "chunk_scan.hpp"
#include "lookback.hpp"
#include "scan_ops.hpp"

namespace linrec {
namespace scan_kernel {

// Waves per SIMD the register budget is set for.  When a compute wave holds at most 32
// floats of chunk data, 7 waves (<= 72 VGPRs) fit without spilling, and a CU holds three of
// the 8-wave workgroups (coordination in wave 0; the SGPR budget allows about 28 waves per
// CU), so one workgroup's look-back hides behind the others' streaming.
// Other shapes (wider chunks, or several channels per lane of WKV or complex pairs, whose
// per-channel state is larger) spill at that budget and keep the compiler's choice.
// The gated WKV instance also holds r per step (80 VGPRs, 6 waves per SIMD): its 8-wave
// workgroups still fit 3 to a CU, as the SGPRs allow no more anyway.
// Operators whose lane offset is used for buffer accesses alone declare kUniformSteps.  For
// them every lane of a wave runs the same step count, and a lane past the last channel gets
// a buffer offset of 2^31, beyond any buffer's range (at most 2^31 - 1 bytes, and row
// offsets stay below 2^31), so its loads return 0 and its stores are dropped by the
// hardware.  The steps' loops then branch on a wave-uniform count instead of a per-lane one
// (B8 T1024 C768 forward: 19.2 -> 18.8 us when measured).
template <class Op, class = void>
struct uniform_steps : std::false_type {};
template <class Op>
struct uniform_steps<Op, std::void_t<decltype(Op::kUniformSteps)>> : std::bool_constant<Op::kUniformSteps> {};
constexpr unsigned kOutOfRange = 0x80000000u;

// Operators that declare kChanLate form their channel constants after the chunk's loads are
// issued (their constants are loads whose wait would hold the chunk's loads back); the
// others form them first (the complex scans' lambda^L, a float64 power, would otherwise wait
// for the whole chunk).
template <class Op, class = void>
struct chan_late : std::false_type {};
template <class Op>
struct chan_late<Op, std::void_t<decltype(Op::kChanLate)>> : std::bool_constant<Op::kChanLate> {};
constexpr int64_t kGridYZMax = 65535;  // grid extent in y and z

template <class Op, int VEC, int L>
constexpr int scan_waves_per_eu() {
    if (std::is_same<Op, WkvExtOp>::value && VEC * L <= 16) return 6;
    return (!Op::kReverse && VEC * L <= 16 && (VEC == 1 || std::is_same<Op, RealOp>::value)) ? 7 : 1;
}

// Addressing of a run of n consecutive logical steps starting at logical step tl of a
// sequence of T: its lowest row (the buffer base) and the Rows of its steps.  Operators in
// reverse time visit the sequence from its last step.
template <bool REV>
__device__ __forceinline__ void run_rows(int64_t T, int64_t tl, int n, unsigned rowb, int64_t& row, Rows& rows) {
    if constexpr (REV) {
        row = n > 0 ? T - tl - n : 0;
        rows = {(unsigned)(n > 0 ? n - 1 : 0) * rowb, -(int)rowb, T - 1 - tl, -1};
    } else {
        row = tl;
        rows = {0u, (int)rowb, tl, 1};
    }
}

// SEP selects where the coordination runs: false, in wave 0, whose chunk is parked in LDS
// meanwhile (NW waves per workgroup); true, in a wave of its own (NW + 1 waves), which
// publishes the inclusive prefix while the chunks re-run.  The first packs more chunks onto
// a CU (it holds about 24 such waves); the second keeps the publication off the chunks'
// path, which pays for long look-back chains of register-heavy operators.
// G3 selects the grid: (ngrp, B, nslab), or a flat one (sizes beyond the 3-D grid's limits).
template <class Op, int VEC, int NW, int L, bool SEP, bool G3>
__global__ __launch_bounds__(64 * (NW + SEP)) __attribute__((amdgpu_waves_per_eu(scan_waves_per_eu<Op, VEC, L>())))
void lookback_scan_kernel(typename Op::Args A, ScanGeom g) {
    using Agg = typename Op::Agg;
    using In = typename Op::In;
    using Chan = typename Op::Chan;
    using Local = typename Op::Local;
    constexpr int CW = 64 * VEC;
    constexpr int SLAB = NW * L;
    constexpr int EF = Op::kFloats;
    constexpr int PL = SEP ? 1 : L;  // parked steps
    using Part = typename Op::Part;
    __shared__ Agg sh[NW][CW];    // chunk aggregates, then sh[x] = chunks 0 .. x-1 combined
    __shared__ Agg sh_carry[CW];  // the carry into the slab
    __shared__ In sh_park[PL][CW];  // wave 0's chunk while it coordinates
    __shared__ Local sh_park_loc[CW];
    __shared__ Part sh_part[Op::kParts ? NW : 1][Op::kParts ? CW : 1];  // chunks' shares of per-slab sums

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    // Slab s (in the recurrence's order: predecessors are dispatched first), batch row b and
    // channel group grp.  A 3-D grid (ngrp, B, nslab) hands them over directly; the flat grid
    // divides the block index, a long scalar sequence that every wave ran before its first
    // load (and whose registers, compiled beside the 3-D path, made the kernels spill SGPRs).
    int64_t s, b, grp;
    if constexpr (G3) {
        s = blockIdx.z;
        b = blockIdx.y;
        grp = blockIdx.x;
    } else {
        const int64_t G = g.B * g.ngrp;
        s = (int64_t)blockIdx.x / G;
        const int64_t gq = (int64_t)blockIdx.x - s * G;
        b = gq / g.ngrp;
        grp = gq - b * g.ngrp;
    }
    const int64_t gi = b * g.ngrp + grp;
    const int64_t c0 = grp * CW + (int64_t)lane * VEC;
    const bool active = c0 < g.C;  // C is a multiple of VEC
    const int64_t t_slab = s * SLAB;
    const int slab_n = (int)((g.T - t_slab) < SLAB ? (g.T - t_slab) : SLAB);
    auto chunk_len = [&](int x) { return max(0, min(L, slab_n - x * L)); };

    // The channels' constants (for WKV w and u; for the complex scans lambda and lambda^L).
    // WKV forms them after the chunk's loads are issued: formed first, their wait held the
    // chunk's loads back by one memory round trip (chan_late).  A lane past the last channel
    // reads the first channels' (no branch around the loads) and keeps the empty constants.
    constexpr bool LATE = chan_late<Op>::value;
    Chan ch[VEC];
    auto form_chan = [&]() {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const Chan x = Op::template chan<L>(A, active ? c0 + e : (int64_t)e);
            ch[e] = active ? x : Chan{};
        }
    };
    if constexpr (!LATE) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) ch[e] = active ? Op::template chan<L>(A, c0 + e) : Chan{};
    }

    const unsigned rowb = (unsigned)(g.C * EF * 4);           // bytes per time step
    constexpr bool UN = uniform_steps<Op>::value;
    // this lane's bytes in the row (out of range for an inactive lane of a uniform-step operator)
    const unsigned voff = (UN && !active) ? kOutOfRange : (unsigned)(lane * VEC * EF * 4);
    const Chain<Agg> chn{g.flags + gi * g.nslab,
                         reinterpret_cast<uint32_t*>(g.rec_agg) + gi * g.nslab * (CW * kRecDwords<Agg>),
                         reinterpret_cast<uint32_t*>(g.rec_incl) + gi * g.nslab * (CW * kRecDwords<Agg>), g.tag, g.spin};
    const bool has_succ = s + 1 < g.nslab;
    // Records in flight per lane in a look-back: fewer for the wide (float64) aggregates.
    constexpr int KB = (VEC >= 4 || kRecDwords<Agg> > 4) ? 2 : (VEC == 2 ? 4 : 8);
    // A chain whose predecessors all fit one batch of records publishes aggregates only
    // (look_back_short); coordination in wave 0 only.
    const bool short_chain = !SEP && g.nslab - 1 <= KB;

    // Coordination, by one whole wave after B1: the slab aggregate (published), the carry
    // into the slab (look-back; into sh_carry), sh[x] = the chunks before x combined (x >= 1).
    // Returns the inclusive prefix, carry followed by the slab.
    auto coordinate = [&](uint64_t first, Agg (&incl)[VEC]) {
        Agg mine[VEC], carry[VEC];
        bool early_carry = false;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            mine[e] = sh[0][lane * VEC + e];
            for (int x = 1; x < NW; ++x) {
                const Agg chunk = sh[x][lane * VEC + e];
                sh[x][lane * VEC + e] = mine[e];
                mine[e] = Op::combine(ch[e], mine[e], chunk, chunk_len(x));
            }
            mine[e] = as_record(mine[e]);  // chain values in the records' form (lookback.hpp)
            carry[e] = as_record(active ? Op::init(A, g, b, c0 + e) : Op::identity());
        }
        auto fold = [&](Agg (&c)[VEC], const Agg (&x)[VEC], int64_t) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) c[e] = as_record(Op::combine(ch[e], c[e], x[e], SLAB));
        };
        // When the flags prefetched before B1 already resolve the carry (every predecessor,
        // or all of them from the nearest inclusive prefix on, published), the slab publishes
        // its inclusive prefix alone: no aggregate, so one store round trip fewer.  The same
        // records in the same association as look_back, so the same bits.  Coordination in
        // wave 0 only: with a coordinator wave of its own (long chains) it measured slower.
        // A short chain publishes aggregates only and folds all of them (look_back_short).
        if (short_chain) {
            early_carry = true;  // carry formed below
        } else if (!SEP && try_look_back<VEC>(chn, s, lane, carry, fold, [] { return true; }, &first)) {
            early_carry = true;
        } else if (has_succ) {
            publish<VEC>(chn, s, lane, mine, false);
        }
        // A slab whose aggregate was not published in time is recomputed from its inputs.
        auto recompute = [&](int64_t jj, Agg (&x)[VEC]) {
            int64_t rowj;
            Rows rj;
            run_rows<Op::kReverse>(g.T, jj * SLAB, SLAB, rowb, rowj, rj);  // predecessors are full slabs
            const typename Op::Res Rj = Op::res(A, g, b, rowj, grp * CW);
#pragma unroll
            for (int e = 0; e < VEC; ++e) x[e] = Op::identity();
            if (active) {
                for (int t = 0; t < SLAB; ++t) {
                    In xi[VEC];
                    Op::template load<VEC>(Rj, voff, rj, t, xi);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) x[e] = Op::step(ch[e], x[e], xi[e]);
                }
            }
#pragma unroll
            for (int e = 0; e < VEC; ++e) x[e] = as_record(x[e]);  // as if read
        };
        if (short_chain) look_back_short<VEC, KB>(chn, s, lane, mine, has_succ, carry, fold, recompute, first);
        else if (!early_carry) look_back<VEC, KB>(chn, s, lane, carry, fold, recompute, first);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            sh_carry[lane * VEC + e] = carry[e];
            incl[e] = as_record(Op::combine(ch[e], carry[e], mine[e], slab_n));
        }
    };
    // Hands the inclusive prefix on: published for the next slab, or, in the last slab, the
    // state after the whole sequence for operators that return it.
    auto hand_on = [&](const Agg (&incl)[VEC]) {
        if (short_chain) {
            if (!has_succ && active) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) Op::finish(A, g, b, c0 + e, incl[e]);
            }
        } else if (has_succ) {
            publish<VEC>(chn, s, lane, incl, true);
        } else if (active) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) Op::finish(A, g, b, c0 + e, incl[e]);
        }
    };
    // The slab's per-slab sum (operators that keep one): the chunks' shares added in order.
    auto slab_sum = [&]() {
        if constexpr (Op::kParts) {
            double re = 0.0, im = 0.0;
            for (int x = 0; x < NW; ++x) {
                re += sh_part[x][lane].re;
                im += sh_part[x][lane].im;
            }
            double* out = g.part + 2 * ((gi * g.nslab + s) * CW + lane);
            out[0] = re;
            out[1] = im;
        }
    };

    if constexpr (SEP) {
        if (w == NW) {
            // ---- the coordinator wave ----
            if constexpr (LATE) form_chan();
            __syncthreads();  // B1: chunk aggregates are in sh
            Agg incl[VEC];
            coordinate(prefetch_window(chn, s, lane), incl);
            __syncthreads();  // B2: the chunks re-run while the inclusive prefix is published
            hand_on(incl);
            if constexpr (Op::kParts) {
                __syncthreads();  // B3: the chunks' shares are in sh_part
                slab_sum();
            }
            return;
        }
    }

    // ---- compute waves: chunk w of the slab, loaded into registers and reduced ----
    const int nu = chunk_len(w);  // steps of the chunk (wave-uniform)
    const int n = (UN || active) ? nu : 0;
    int64_t row;
    Rows rows;
    run_rows<Op::kReverse>(g.T, t_slab + (int64_t)w * L, nu, rowb, row, rows);
    const typename Op::Res R = Op::res(A, g, b, row, grp * CW);
    In in[L][VEC];
    if (n == L) {
#pragma unroll
        for (int j = 0; j < L; ++j) Op::template load<VEC>(R, voff, rows, j, in[j]);
    } else {
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < n) Op::template load<VEC>(R, voff, rows, j, in[j]);
            else Op::template zero<VEC>(in[j]);
        }
    }
    if constexpr (LATE) form_chan();
    Local loc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) sh[w][lane * VEC + e] = Op::template reduce<L, VEC>(ch[e], in, e, n, loc[e]);
    if (SEP || w != 0) {
        __syncthreads();  // B1: chunk aggregates are in sh
        __syncthreads();  // B2: the slab's carry is in sh_carry, every chunk's prefix in sh[w]
    } else {
        // Wave 0 coordinates.  Its chunk waits in LDS meanwhile, and the whole role sits in
        // this one branch, so that the look-back's registers do not add to the chunk's.
#pragma unroll
        for (int j = 0; j < PL; ++j)
#pragma unroll
            for (int e = 0; e < VEC; ++e) sh_park[j][lane * VEC + e] = in[j][e];
#pragma unroll
        for (int e = 0; e < VEC; ++e) sh_park_loc[lane * VEC + e] = loc[e];
        const uint64_t first = prefetch_window(chn, s, lane);  // overlaps the wait at B1
        __syncthreads();  // B1
        Agg incl[VEC];
        coordinate(first, incl);
        hand_on(incl);
        __syncthreads();  // B2
#pragma unroll
        for (int j = 0; j < PL; ++j)
#pragma unroll
            for (int e = 0; e < VEC; ++e) in[j][e] = sh_park[j][lane * VEC + e];
#pragma unroll
        for (int e = 0; e < VEC; ++e) loc[e] = sh_park_loc[lane * VEC + e];
    }

    // ---- re-run the chunk from its carry ----
    Part part{};
    if (n > 0) {
        Agg cin[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            cin[e] = (w == 0) ? sh_carry[lane * VEC + e]
                              : Op::combine(ch[e], sh_carry[lane * VEC + e], sh[w][lane * VEC + e], w * L);
        part = Op::template run<L, VEC>(R, ch, cin, in, loc, n, voff, rows);
    }
    if constexpr (Op::kParts) {
        static_assert(VEC == 1, "per-slab sums are kept for one channel per lane");
        sh_part[w][lane] = part;
        __syncthreads();  // B3: the chunks' shares are in sh_part
        if (!SEP && w == 0) slab_sum();
    }
}

template <class Op, int VEC, int NW, int L>
hipError_t launch(const typename Op::Args& A, const ScanGeom& g, bool sep, hipStream_t st) {
    const int64_t nb = g.B * g.ngrp * g.nslab;
    if (const hipError_t e = clear_flags_if_capturing(g.flags, nb, st)) return e;
    // The 3-D grid numbers blocks x fastest, then y, then z: the same slab-major order as the
    // flat one.  Its y and z extents are kept within 65535.  Kernels with a coordinator wave of
    // their own (the complex scans: long chains, many rounds of workgroups) keep the flat grid,
    // which measured faster for them (B1 T262144 C1024 LRU scan 764 vs 776 us); for the others
    // the 3-D grid saves the prologue's divisions.
    // LINREC_FLAT_GRID=1 takes the flat grid at any size (tests).
    const char* flat = std::getenv("LINREC_FLAT_GRID");
    const bool g3 = g.B <= kGridYZMax && g.nslab <= kGridYZMax && !(flat && flat[0] == '1');
    const dim3 grid3((unsigned)g.ngrp, (unsigned)g.B, (unsigned)g.nslab), grid1((unsigned)nb);
    if constexpr (VEC == 1) {
        if (sep) {
            hipLaunchKernelGGL((lookback_scan_kernel<Op, VEC, NW, L, true, false>), grid1, dim3(64 * (NW + 1)), 0, st,
                               A, g);
            return hipGetLastError();
        }
    }
    if (g3)
        hipLaunchKernelGGL((lookback_scan_kernel<Op, VEC, NW, L, false, true>), grid3, dim3(64 * NW), 0, st, A, g);
    else
        hipLaunchKernelGGL((lookback_scan_kernel<Op, VEC, NW, L, false, false>), grid1, dim3(64 * NW), 0, st, A, g);
    return hipGetLastError();
}

// Kernels that exist: vec in {VMAX, 2, 1} x (nw, L) in {(4, 16), (8, 8), (8, 16)}, and for
// the linear scans (8, 32) with one channel per lane (the registers of two channels x 16
// steps, with slabs twice as long: shorter look-back chains); each with the coordination in
// wave 0, and for one channel per lane also with a coordinator wave.  WKV keeps chunks of at
// most 16 steps: its per-chunk frame spans (L-1) om in exponent, which 32 steps of a fast
// decay push to the edge of float32 range.
template <class Op, int VEC>
hipError_t dispatch_shape(const typename Op::Args& A, const ScanGeom& g, const ScanPlan& p, hipStream_t st) {
    if (p.nw == 4 && p.L == 16) return launch<Op, VEC, 4, 16>(A, g, p.sep, st);
    if (p.nw == 8 && p.L == 8) return launch<Op, VEC, 8, 8>(A, g, p.sep, st);
    if (p.nw == 8 && p.L == 16) return launch<Op, VEC, 8, 16>(A, g, p.sep, st);
    if constexpr (VEC == 1 && !std::is_same<Op, WkvOp>::value && !std::is_same<Op, WkvExtOp>::value) {
        if (p.nw == 8 && p.L == 32) return launch<Op, VEC, 8, 32>(A, g, p.sep, st);
    }
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

}  // namespace scan_kernel
}  // namespace linrec

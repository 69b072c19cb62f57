// lookback.hpp -- decoupled look-back over the slabs of one sequence (device code, internal).
//
// A sequence is cut into slabs that the recurrence visits in a fixed order, the chain
// (q = 0 first: time order for a forward scan, reverse time order for a backward one).  Each
// slab publishes its aggregate (AGG), then -- once it knows its carry-in -- its inclusive
// prefix (INCL); a slab that knows its carry before its aggregate is formed may publish
// INCL alone (its flag never reads AGG, so no reader looks for the missing record).  A slab's
// carry is the nearest published INCL folded with the aggregates of the slabs after it, in
// chain order: the association a strictly chained scan would use, so the result does not
// depend on timing.  That needs every INCL_q to equal, bit for bit, INCL_{q-1} folded with
// AGG_q as a reader would fold them: a publisher forms INCL as its carry folded with the
// very aggregate it publishes, and where records are narrower than the aggregates every
// chain value (aggregate, each fold, INCL) is taken in the record's form (as_record).
//
// Records are written and read with device-scope relaxed atomics, which the hardware keeps
// coherent across the XCDs' L2 caches (they write through), and a publication flag is
// stored only after all of the wave's record stores have completed (s_waitcnt).  This
// avoids agent-scope release/acquire fences, whose L2 writeback or invalidation serialises
// per XCD.  Records are stored field-major -- dword i of entry (e, lane) of slab q at
// ((q * ND + i) * VEC + e) * 64 + lane -- so each of those one-dword stores covers 256
// contiguous bytes and writes whole lines through to memory.
//
// Every wait is bounded: a slab whose flag has not appeared after `spin` polls is
// recomputed from its inputs by the waiting wave.  Flags carry a per-call tag, so stale
// flags from earlier calls read as "not published" and the workspace needs no clearing.
#pragma once

#include "device_common.hpp"

namespace linrec {

constexpr uint64_t kStateAgg = 1;  // flag = tag * 4 + state
constexpr uint64_t kStateIncl = 2;

template <class Agg>
constexpr int kDwords = (int)(sizeof(Agg) / 4);

// The form a record takes in memory: the aggregate itself, unless its type names a narrower
// one (a specialisation of RecordOf) that every publisher and every reader converts through,
// so that all of them fold the same values.
template <class Agg>
struct RecordOf {
    using type = Agg;
    __device__ __forceinline__ static Agg to(const Agg& a) { return a; }
    __device__ __forceinline__ static Agg from(const Agg& r) { return r; }
};
template <class Agg>
constexpr int kRecDwords = kDwords<typename RecordOf<Agg>::type>;

// x as a record holds it (x itself unless Agg has a narrower record form); idempotent.
template <class Agg>
__device__ __forceinline__ Agg as_record(const Agg& x) {
    return RecordOf<Agg>::from(RecordOf<Agg>::to(x));
}

// This wave's VEC entries per lane of slab q's record (rec: dwords, field-major).
template <int VEC, class Agg>
__device__ __forceinline__ void store_record(uint32_t* rec, int64_t q, int lane, const Agg (&x)[VEC]) {
    using Rec = typename RecordOf<Agg>::type;
    static_assert(sizeof(Rec) % 4 == 0, "record must be whole dwords");
    constexpr int ND = kDwords<Rec>;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        uint32_t w[ND];
        const Rec r = RecordOf<Agg>::to(x[e]);
        __builtin_memcpy(w, &r, sizeof(Rec));
#pragma unroll
        for (int i = 0; i < ND; ++i)
            __hip_atomic_store(rec + ((q * ND + i) * VEC + e) * 64 + lane, w[i], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int VEC, class Agg>
__device__ __forceinline__ void load_record(const uint32_t* rec, int64_t q, int lane, Agg (&x)[VEC]) {
    using Rec = typename RecordOf<Agg>::type;
    constexpr int ND = kDwords<Rec>;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        uint32_t w[ND];
#pragma unroll
        for (int i = 0; i < ND; ++i)
            w[i] = __hip_atomic_load(rec + ((q * ND + i) * VEC + e) * 64 + lane, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
        Rec r;
        __builtin_memcpy(&r, w, sizeof(Rec));
        x[e] = RecordOf<Agg>::from(r);
    }
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

// The records of one sequence's chain: slab q owns flags[q] and the 64 * VEC entries of
// agg and incl at slab index q (dword arrays, field-major).
template <class Agg>
struct Chain {
    uint64_t* flags;
    uint32_t* agg;
    uint32_t* incl;
    uint64_t tag;
    int spin;
};

// Publish this wave's VEC records per lane for slab q as its aggregate or inclusive prefix.
template <int VEC, class Agg>
__device__ __forceinline__ void publish(const Chain<Agg>& ch, int64_t q, int lane, const Agg (&x)[VEC],
                                        bool inclusive) {
    store_record<VEC>(inclusive ? ch.incl : ch.agg, q, lane, x);
    wait_memory();
    if (lane == 0)
        __hip_atomic_store(ch.flags + q, ch.tag * 4 + (inclusive ? kStateIncl : kStateAgg), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Carry into chain slab q, computed by one whole wave.  On entry `carry` holds the state
// before chain slab 0; on return, the state before slab q:
//   fold(carry, x, j)    carry <- carry followed by slab j whose aggregate is x;
//   recompute(j, x)      x <- slab j's aggregate, computed from its inputs.
// `first` is the optional result of prefetch_window for the first round.
// Phase A: lane i inspects slab hi-1-i, 64 predecessors per round trip, until a round finds
// a published inclusive prefix (the nearest one, j0) or slab 0 is passed (j0 = -1); lanes
// remember which slabs had published.  Phase B: carry = INCL_j0 (or the entry state) folded
// with the aggregates of slabs j0+1 .. q-1, fetched KB slabs at a time (issued together,
// then folded in order) so the fold costs one memory round trip per KB slabs.
// One relaxed read of the flag of slab q-1-lane (the first look-back window), issued early
// so that its round trip overlaps other work; look_back takes it as `first`.
template <class Agg>
__device__ __forceinline__ uint64_t prefetch_window(const Chain<Agg>& ch, int64_t q, int lane) {
    const int64_t j = q - 1 - lane;
    return j >= 0 ? __hip_atomic_load(ch.flags + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
}

template <int VEC, int KB, class Agg, class Fold, class Recompute>
__device__ __forceinline__ void look_back(const Chain<Agg>& ch, int64_t q, int lane, Agg (&carry)[VEC],
                                          Fold&& fold, Recompute&& recompute, uint64_t first = 0) {
    constexpr int kWin = 16;  // windows whose publication masks are kept
    uint64_t pub[kWin];
#pragma unroll
    for (int x = 0; x < kWin; ++x) pub[x] = 0;
    int64_t j0 = -1;
    int nwin = 0;
    for (int64_t hi = q; hi > 0; hi -= 64, ++nwin) {
        const int64_t j = hi - 1 - lane;
        // A flag already seen published in the prefetched first window is final.
        const bool have = nwin == 0 && (first >> 2) == ch.tag;
        const uint64_t f = (j >= 0) ? (have ? first : poll_flag(ch.flags + j, ch.tag, ch.spin)) : 0;
        const uint64_t incl_mask = __ballot(j >= 0 && f == ch.tag * 4 + kStateIncl);
        const uint64_t pub_mask = __ballot(j >= 0 && (f >> 2) == ch.tag);
#pragma unroll
        for (int x = 0; x < kWin; ++x)
            if (x == nwin) pub[x] = pub_mask;
        if (incl_mask) {
            j0 = hi - 1 - (int64_t)(__ffsll((long long)incl_mask) - 1);
            break;
        }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);  // record loads stay after the polls
    if (j0 >= 0) load_record<VEC>(ch.incl, j0, lane, carry);
    for (int64_t j = j0 + 1; j < q; j += KB) {
        Agg xb[KB][VEC];
        bool pubb[KB], inclb[KB];
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const int64_t jj = j + k;
            pubb[k] = inclb[k] = false;
            if (jj < q) {
                const int64_t back = q - 1 - jj;  // lane index of slab jj in its window
                const int x = (int)(back >> 6);
                if (x < kWin) {
                    uint64_t m = 0;
#pragma unroll
                    for (int y = 0; y < kWin; ++y)
                        if (y == x) m = pub[y];
                    pubb[k] = (m >> (back & 63)) & 1;
                } else {
                    // Beyond the remembered windows the flag is read again.  A slab may
                    // publish its inclusive prefix without an aggregate (a writer that knew
                    // its carry early); one seen now replaces the carry folded so far, which
                    // it extends in the same association.
                    const uint64_t f = first_lane_u64((lane == 0) ? poll_flag(ch.flags + jj, ch.tag, ch.spin) : 0);
                    pubb[k] = (f >> 2) == ch.tag;
                    inclb[k] = f == ch.tag * 4 + kStateIncl;
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
                }
                if (pubb[k]) load_record<VEC>(inclb[k] ? ch.incl : ch.agg, jj, lane, xb[k]);
            }
        }
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const int64_t jj = j + k;
            if (jj < q) {
                if (inclb[k]) {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) carry[e] = xb[k][e];
                } else {
                    if (!pubb[k]) recompute(jj, xb[k]);  // not published in time
                    fold(carry, xb[k], jj);
                }
            }
        }
    }
}

// Look-back over a short chain (q <= KB: all predecessors in one batch), in which every slab
// publishes its aggregate alone and a slab's carry is the entry state folded with the
// aggregates of all its predecessors, in chain order (the same association whatever the
// timing).  The slab's own record stores (when it has a successor) and its predecessors'
// record loads are in flight together, so a slab whose predecessors had published when
// their flags were prefetched (`first`, see prefetch_window) pays one memory round trip
// where publishing an inclusive prefix after the carry costs two.  When some predecessor
// has not published yet, the slab raises its own flag first, then polls.
template <int VEC, int KB, class Agg, class Fold, class Recompute>
__device__ __forceinline__ void look_back_short(const Chain<Agg>& ch, int64_t q, int lane, const Agg (&mine)[VEC],
                                                bool publish_mine, Agg (&carry)[VEC], Fold&& fold,
                                                Recompute&& recompute, uint64_t first) {
    static_assert(KB < 64, "one window of flags");
    auto raise = [&]() {
        wait_memory();  // the records have been performed before the flag is stored
        if (lane == 0)
            __hip_atomic_store(ch.flags + q, ch.tag * 4 + kStateAgg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    if (publish_mine) store_record<VEC>(ch.agg, q, lane, mine);
    const int64_t j = q - 1 - lane;  // lane i watches slab q-1-i
    const uint64_t need = (1ull << q) - 1;
    uint64_t f = (j >= 0) ? first : 0;
    uint64_t pub = __ballot(j >= 0 && (f >> 2) == ch.tag);
    bool raised = false;
    if ((pub & need) != need) {
        // The missing flags are read again while this slab's records are being stored (one
        // round trip for both), then polled if still missing.
        if (j >= 0 && (f >> 2) != ch.tag) f = __hip_atomic_load(ch.flags + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (publish_mine) raise();
        raised = true;
        if (j >= 0 && (f >> 2) != ch.tag) f = poll_flag(ch.flags + j, ch.tag, ch.spin);
        pub = __ballot(j >= 0 && (f >> 2) == ch.tag);
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);  // record loads stay after the polls
    Agg xb[KB][VEC];
#pragma unroll
    for (int k = 0; k < KB; ++k)
        if (k < q && ((pub >> (q - 1 - k)) & 1)) load_record<VEC>(ch.agg, k, lane, xb[k]);
    if (publish_mine && !raised) raise();
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        if (k < q) {
            if (!((pub >> (q - 1 - k)) & 1)) recompute((int64_t)k, xb[k]);  // not published in time
            fold(carry, xb[k], (int64_t)k);
        }
    }
}

// A non-blocking attempt at look_back's result, for a coordinator that would otherwise sit
// idle while its workgroup's other waves work: polls the flags of the 64 nearest
// predecessors until they hold a published inclusive prefix with every aggregate after it
// published (or, for q <= 64, every predecessor's aggregate), then folds exactly as
// look_back does -- same records, same association, so the same bits -- and returns true.
// Returns false, with `carry` untouched, as soon as give_up() holds or after ch.spin polls;
// the caller then publishes its aggregate and calls look_back.  Chains longer than 64 slabs
// without an inclusive prefix in that window always end that way.  With `first` (the
// prefetched window of prefetch_window), the first round reads those flags instead of
// polling again.
template <int VEC, class Agg, class Fold, class GiveUp>
__device__ __forceinline__ bool try_look_back(const Chain<Agg>& ch, int64_t q, int lane, Agg (&carry)[VEC],
                                              Fold&& fold, GiveUp&& give_up, const uint64_t* first = nullptr) {
    if (q == 0) return true;
    const int64_t j = q - 1 - lane;  // lane i watches slab q-1-i
    for (int it = 0;; ++it) {
        const uint64_t f = j < 0 ? 0
                           : (it == 0 && first) ? *first
                                                : __hip_atomic_load(ch.flags + j, __ATOMIC_RELAXED,
                                                                    __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t incl_mask = __ballot(j >= 0 && f == ch.tag * 4 + kStateIncl);
        const uint64_t pub_mask = __ballot(j >= 0 && (f >> 2) == ch.tag);
        bool ready = false;
        int64_t j0 = -1;
        if (incl_mask) {
            const int i0 = __ffsll((long long)incl_mask) - 1;  // the nearest inclusive prefix
            const uint64_t need = i0 == 0 ? 0ull : ((1ull << i0) - 1);
            ready = (pub_mask & need) == need;
            j0 = q - 1 - i0;
        } else if (q <= 64) {
            const uint64_t need = q == 64 ? ~0ull : ((1ull << q) - 1);
            ready = (pub_mask & need) == need;
        }
        if (ready) {
            __atomic_signal_fence(__ATOMIC_SEQ_CST);  // record loads stay after the polls
            if (j0 >= 0) load_record<VEC>(ch.incl, j0, lane, carry);
            for (int64_t jj = j0 + 1; jj < q; ++jj) {
                Agg x[VEC];
                load_record<VEC>(ch.agg, jj, lane, x);
                fold(carry, x, jj);
            }
            return true;
        }
        if (give_up() || it >= ch.spin) return false;
        __builtin_amdgcn_s_sleep(2);
    }
}

}  // namespace linrec

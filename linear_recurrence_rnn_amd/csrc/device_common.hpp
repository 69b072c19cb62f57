// device_common.hpp -- small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace linrec {

// log2(e): the WKV kernels work in base 2 so every exponential is one v_exp_f32.
constexpr float kLog2e = 1.4426950408889634f;
// Log-scale of an empty WKV state.  Finite so that "empty - empty" is 0, not NaN;
// 2^(kEmpty - x) is exactly 0 for every x a real state can hold.
constexpr float kEmpty = -1.0e30f;
// MI355X: 8 accelerator complex dies; consecutive workgroups go to consecutive XCDs.
constexpr int kNumXcd = 8;

// Map the hardware block index to a logical one so that each XCD (and its private L2)
// receives one contiguous range of logical blocks: neighbouring channel groups, which
// share 128-byte lines, then run on the same L2.  A bijection on [0, nb).
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t nb) {
    const int64_t xcd = bid % kNumXcd, local = bid / kNumXcd;
    const int64_t per = nb / kNumXcd, rem = nb % kNumXcd;
    return xcd * per + (xcd < rem ? xcd : rem) + local;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Native clang vectors: what the nontemporal load/store builtins accept.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// N consecutive floats at p (p aligned to 4*N bytes for N = 2, 4; 16 bytes for N = 8).
// Streaming data is read and written once, so the accesses are marked nontemporal.
template <int N> struct FV { float v[N]; };

template <int N>
__device__ __forceinline__ FV<N> ldg(const float* __restrict__ p) {
    FV<N> r;
    if constexpr (N == 1) {
        r.v[0] = __builtin_nontemporal_load(p);
    } else if constexpr (N == 2) {
        const f32x2 t = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(p));
        r.v[0] = t.x; r.v[1] = t.y;
    } else if constexpr (N == 4) {
        const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
        r.v[0] = t.x; r.v[1] = t.y; r.v[2] = t.z; r.v[3] = t.w;
    } else {
        static_assert(N == 8, "unsupported vector width");
        const f32x4 t0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
        const f32x4 t1 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
        r.v[0] = t0.x; r.v[1] = t0.y; r.v[2] = t0.z; r.v[3] = t0.w;
        r.v[4] = t1.x; r.v[5] = t1.y; r.v[6] = t1.z; r.v[7] = t1.w;
    }
    return r;
}

template <int N>
__device__ __forceinline__ void stg(float* __restrict__ p, const FV<N>& r) {
    if constexpr (N == 1) {
        __builtin_nontemporal_store(r.v[0], p);
    } else if constexpr (N == 2) {
        const f32x2 t = {r.v[0], r.v[1]};
        __builtin_nontemporal_store(t, reinterpret_cast<f32x2*>(p));
    } else if constexpr (N == 4) {
        const f32x4 t = {r.v[0], r.v[1], r.v[2], r.v[3]};
        __builtin_nontemporal_store(t, reinterpret_cast<f32x4*>(p));
    } else {
        static_assert(N == 8, "unsupported vector width");
        const f32x4 t0 = {r.v[0], r.v[1], r.v[2], r.v[3]};
        const f32x4 t1 = {r.v[4], r.v[5], r.v[6], r.v[7]};
        __builtin_nontemporal_store(t0, reinterpret_cast<f32x4*>(p));
        __builtin_nontemporal_store(t1, reinterpret_cast<f32x4*>(p) + 1);
    }
}

// ---- buffer addressing ----------------------------------------------------------
// Streaming tensors are addressed through a buffer resource per wave: a scalar base
// pointer (uniform per wave), a 32-bit per-lane byte offset and a scalar per-step offset,
// instead of one 64-bit address per load.  Accesses at or beyond num_records return 0
// (loads) or are dropped (stores).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufNT = 2;  // cache policy: non-temporal (streamed once)

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t nbytes) {
    const int n = nbytes > 0x7fffffff ? 0x7fffffff : (nbytes < 0 ? 0 : (int)nbytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

template <int N>
__device__ __forceinline__ FV<N> ldb(rsrc_t rs, unsigned voff, unsigned soff) {
    FV<N> r;
    if constexpr (N == 1) {
        r.v[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, kBufNT));
    } else if constexpr (N == 2) {
        const f32x2 t = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, kBufNT));
        r.v[0] = t.x; r.v[1] = t.y;
    } else if constexpr (N == 4) {
        const f32x4 t = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, kBufNT));
        r.v[0] = t.x; r.v[1] = t.y; r.v[2] = t.z; r.v[3] = t.w;
    } else {
        static_assert(N == 8, "unsupported vector width");
        const f32x4 t0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, kBufNT));
        const f32x4 t1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16, soff, kBufNT));
        r.v[0] = t0.x; r.v[1] = t0.y; r.v[2] = t0.z; r.v[3] = t0.w;
        r.v[4] = t1.x; r.v[5] = t1.y; r.v[6] = t1.z; r.v[7] = t1.w;
    }
    return r;
}

template <int N>
__device__ __forceinline__ void stb(rsrc_t rs, unsigned voff, unsigned soff, const FV<N>& r) {
    if constexpr (N == 1) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, r.v[0]), rs, voff, soff, kBufNT);
    } else if constexpr (N == 2) {
        const f32x2 t = {r.v[0], r.v[1]};
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, t), rs, voff, soff, kBufNT);
    } else if constexpr (N == 4) {
        const f32x4 t = {r.v[0], r.v[1], r.v[2], r.v[3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, t), rs, voff, soff, kBufNT);
    } else {
        static_assert(N == 8, "unsupported vector width");
        const f32x4 t0 = {r.v[0], r.v[1], r.v[2], r.v[3]};
        const f32x4 t1 = {r.v[4], r.v[5], r.v[6], r.v[7]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, t0), rs, voff, soff, kBufNT);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, t1), rs, voff + 16, soff, kBufNT);
    }
}

}  // namespace linrec

// part_reduce.hpp -- dL/dlambda of the decay and LRU adjoints: the sum over slabs and batch
// rows of the per-slab, per-channel shares the scan kernel leaves in g.part, as two small
// kernels after the scan (device code, internal).
//
// dL/dlambda is a sum over batch and time of per-step terms (the chain rule of the
// recurrence: the LRU write-up's diagonal recurrence, and the real decay).  The scan's
// workgroups each add their own slab's steps; these kernels add the shares in two stages
// whose association is fixed by index alone, so the bits do not depend on scheduling:
//   stage 1  (part_sum_kernel) for each batch row b and block k of kPartBlock consecutive
//            slabs (chain order), the shares, slab i of the block to accumulator i mod 8,
//            in ascending i, then the 8 accumulators in order;
//   stage 2  (part_final_kernel) for each channel, the stage-1 sums of every (b, k), entry
//            e = b * nk + k to accumulator e mod 8 in ascending e, then the accumulators in
//            order, written as float32 (or complex64).
// Each of a workgroup's 8 waves owns one accumulator and issues all of its loads at once,
// so a stage costs one round of loads (per 64 entries).
// Measured alternatives, both slower on MI355X: the shares summed inside the scan kernel by
// the last-arriving workgroup (each slab's workgroup then waits for its share's store and
// a counter update before it retires), and one kernel whose last workgroup runs stage 2.
#pragma once

#include "chunk_scan.hpp"

namespace linrec {

constexpr int kPartWaves = 8;  // one accumulator per wave

// Accumulator w of one stage: the sum over entries i = w, w + 8, ... < n (ascending) of the
// pairs at x + i * stride, each round's loads issued before its adds.
__device__ __forceinline__ void part_accumulate(const double* x, int64_t stride, int64_t n, int w, double& re,
                                                double& im) {
    constexpr int kMax = kPartBlock / kPartWaves;  // entries per wave in one round
    re = im = 0.0;
    for (int64_t i0 = w; i0 < n; i0 += (int64_t)kMax * kPartWaves) {
        double vr[kMax], vi[kMax];
#pragma unroll
        for (int m = 0; m < kMax; ++m) {
            const int64_t i = i0 + (int64_t)m * kPartWaves;
            vr[m] = vi[m] = 0.0;
            if (i < n) {
                vr[m] = x[i * stride];
                vi[m] = x[i * stride + 1];
            }
        }
#pragma unroll
        for (int m = 0; m < kMax; ++m) {
            if (i0 + (int64_t)m * kPartWaves < n) {
                re += vr[m];
                im += vi[m];
            }
        }
    }
}

// The 8 waves' accumulators of lane's channel, added in order (valid in wave 0).
__device__ __forceinline__ void part_combine(double (&sh)[kPartWaves][64][2], int w, int lane, double re, double im,
                                             double& r, double& i) {
    sh[w][lane][0] = re;
    sh[w][lane][1] = im;
    __syncthreads();
    r = i = 0.0;
    if (w == 0) {
        for (int x = 0; x < kPartWaves; ++x) {
            r += sh[x][lane][0];
            i += sh[x][lane][1];
        }
    }
}

// Stage 1: grid (ngrp, nk, min(B, 65535)), 64 * kPartWaves threads.
__global__ __launch_bounds__(64 * kPartWaves) void part_sum_kernel(ScanGeom g) {
    __shared__ double sh[kPartWaves][64][2];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t grp = blockIdx.x, k = blockIdx.y;
    const int64_t c = grp * 64 + lane;
    const bool active = c < g.C;
    const int64_t s0 = k * kPartBlock, n1 = (g.nslab - s0) < kPartBlock ? (g.nslab - s0) : kPartBlock;
    for (int64_t b = blockIdx.z; b < g.B; b += gridDim.z) {  // uniform over the workgroup
        const int64_t gi = b * g.ngrp + grp;
        double re, im, r1, i1;
        part_accumulate(g.part + 2 * ((gi * g.nslab + s0) * 64 + lane), 2 * 64, active ? n1 : 0, w, re, im);
        part_combine(sh, w, lane, re, im, r1, i1);
        if (w == 0 && active) {
            g.part2[2 * ((b * g.nk + k) * g.C + c)] = r1;
            g.part2[2 * ((b * g.nk + k) * g.C + c) + 1] = i1;
        }
        __syncthreads();  // sh is reused by the next row
    }
}

// Stage 2: grid (ngrp), 64 * kPartWaves threads.  glam: C complex64 (complex_out) or C
// float32 (the real parts).
__global__ __launch_bounds__(64 * kPartWaves) void part_final_kernel(ScanGeom g, float* __restrict__ glam,
                                                                      bool complex_out) {
    __shared__ double sh[kPartWaves][64][2];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t c = (int64_t)blockIdx.x * 64 + lane;
    const bool active = c < g.C;
    double re, im, r2, i2;
    part_accumulate(g.part2 + 2 * c, 2 * g.C, active ? g.B * g.nk : 0, w, re, im);
    part_combine(sh, w, lane, re, im, r2, i2);
    if (w == 0 && active) {
        if (complex_out) {
            glam[2 * c] = (float)r2;
            glam[2 * c + 1] = (float)i2;
        } else {
            glam[c] = (float)r2;
        }
    }
}

}  // namespace linrec

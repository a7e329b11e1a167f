// Block-wide (256 threads) helpers for drawing an index by inverse CDF over
// non-negative weights held in LDS: sums, and the first index at which the
// running sum passes a target.
#pragma once
#include <hip/hip_runtime.h>

namespace aw4 {

// LDS the helpers need: 4 wave totals + 4 reduction slots
struct BlockScanLds {
    float wave_tot[4];
    int ired[4];
    float fred[4];
};

__device__ __forceinline__ int block_min_int(int v, BlockScanLds& s) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) s.ired[threadIdx.x >> 6] = v;
    __syncthreads();
    return min(min(s.ired[0], s.ired[1]), min(s.ired[2], s.ired[3]));
}

__device__ __forceinline__ int block_max_int(int v, BlockScanLds& s) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) s.ired[threadIdx.x >> 6] = v;
    __syncthreads();
    return max(max(s.ired[0], s.ired[1]), max(s.ired[2], s.ired[3]));
}

// Sum of w[0..n) (n <= 256 PER), the same fixed order in every call.
template <int PER>
__device__ __forceinline__ float block_sum_lds(const float* w, int n, BlockScanLds& s) {
    const int i0 = threadIdx.x * PER;
    float v = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e)
        if (i0 + e < n) v += w[i0 + e];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) s.fred[threadIdx.x >> 6] = v;
    __syncthreads();
    return (s.fred[0] + s.fred[1]) + (s.fred[2] + s.fred[3]);
}

// Inverse CDF over w[0..n) in LDS (n <= 256 PER): the smallest i with
// base + w[0] + ... + w[i] > target and w[i] > 0; if rounding leaves no such i,
// the last i with w[i] > 0; -1 if every weight is 0.  Thread t owns elements
// [t PER, t PER + PER) and adds them in order after an exclusive scan of the
// per-thread sums.  *before receives base plus the weights ahead of the
// returned index.  Every thread of the block must call it; the result is
// uniform.
template <int PER>
__device__ __forceinline__ int block_inverse_cdf(const float* w, int n, float base, float target, float* before,
                                                 BlockScanLds& s) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i0 = tid * PER;
    float loc = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e)
        if (i0 + e < n) loc += w[i0 + e];
    // inclusive scan of the per-thread sums inside the wave, then across waves
    float inc = loc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float u = __shfl_up(inc, o, 64);
        if (lane >= o) inc += u;
    }
    __syncthreads();
    if (lane == 63) s.wave_tot[wave] = inc;
    __syncthreads();
    float run = base + (inc - loc);
    for (int k = 0; k < wave; ++k) run += s.wave_tot[k];
    int hit = 0x7fffffff, last = -1;
    float hit_before = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int i = i0 + e;
        if (i < n) {
            const float wi = w[i];
            if (wi > 0.f) last = i;
            if (hit == 0x7fffffff && wi > 0.f && run + wi > target) {
                hit = i;
                hit_before = run;
            }
            run += wi;
        }
    }
    const int first = block_min_int(hit, s);
    if (first != 0x7fffffff) {
        if (hit == first) *before = hit_before;
        __syncthreads();
        return first;
    }
    const int lastnz = block_max_int(last, s);
    if (lastnz >= 0 && lastnz >= i0 && lastnz < i0 + PER) {
        float r = base + (inc - loc);
        for (int k = 0; k < wave; ++k) r += s.wave_tot[k];
        for (int i = i0; i < lastnz; ++i) r += w[i];
        *before = r;
    }
    __syncthreads();
    return lastnz;
}

}  // namespace aw4

// W4A16 dequant-GEMV and the int8 output head for gfx950.
//
// Decode reads every weight once per token (page 5, bs178.com llamAmpere
// article, "为什么它真能这么快" point 二: single-token generation is bandwidth
// bound), so these kernels are built around streaming the packed codes with
// coalesced loads and doing as little VALU work per weight as possible.
//
// Layout of work: one wavefront owns a pair of output rows; its 64 lanes walk
// the row in 16-weight chunks (8 bytes of codes per lane per row, so a wave
// load covers 512 contiguous bytes), dot each chunk with the fp16 input held
// in LDS, scale the chunk by its group's fp16 scale and reduce across lanes.
// The input vector is produced by a fused prologue (RMSNorm, gated RMSNorm or
// a plain fp16 load) and the result leaves through a fused epilogue (store,
// residual add, SwiGLU of an interleaved gate/up pair).
#include <mutex>

#include "aw4_internal.h"

#include <algorithm>

namespace aw4 {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }

// 8 nibbles of one dword (slot order [0,2,4,6,1,3,5,7]) against x[0..7] given
// as four fp16 pairs.  Each nibble n is placed in the mantissa of fp16 1024
// (0x6400 | n = 1024 + n, or 1024 + 16 n for the upper nibble of a byte) and
// the offset is removed with one packed subtraction: exact codes c = n - 8,
// the upper-nibble ones scaled by 16.
__device__ __forceinline__ void dq_dot8(uint32_t w, uint4 xv, float& ea, float& eb) {
    const h2 off_lo = {(_Float16)1032.0f, (_Float16)1032.0f};
    const h2 off_hi = {(_Float16)1152.0f, (_Float16)1152.0f};
    uint32_t w8 = w >> 8;
    h2 p0 = as_h2((w & 0x000F000Fu) | 0x64006400u) - off_lo;
    h2 p1 = as_h2((w & 0x00F000F0u) | 0x64006400u) - off_hi;
    h2 p2 = as_h2((w8 & 0x000F000Fu) | 0x64006400u) - off_lo;
    h2 p3 = as_h2((w8 & 0x00F000F0u) | 0x64006400u) - off_hi;
    ea = __builtin_amdgcn_fdot2(p0, as_h2(xv.x), ea, false);
    eb = __builtin_amdgcn_fdot2(p1, as_h2(xv.y), eb, false);
    ea = __builtin_amdgcn_fdot2(p2, as_h2(xv.z), ea, false);
    eb = __builtin_amdgcn_fdot2(p3, as_h2(xv.w), eb, false);
}

// The same with the constants where a VOP3 can read them (gfx9 VOP3 encodings
// take no literals): masks in SGPRs and the exponent pattern in a VGPR, so each
// (w & mask) | 0x6400 pair is one v_and_or_b32 instead of an and plus an or.
struct NibK {
    uint32_t lo, hi, e;
    __device__ __forceinline__ NibK() {
        asm volatile("s_mov_b32 %0, 0xf000f" : "=s"(lo));
        asm volatile("s_mov_b32 %0, 0xf000f0" : "=s"(hi));
        asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(e));
    }
};
__device__ __forceinline__ void dq_dot8(uint32_t w, uint4 xv, float& ea, float& eb, const NibK& k) {
    const h2 off_lo = {(_Float16)1032.0f, (_Float16)1032.0f};
    const h2 off_hi = {(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t w8 = w >> 8;
    const h2 p0 = as_h2((w & k.lo) | k.e) - off_lo;
    const h2 p1 = as_h2((w & k.hi) | k.e) - off_hi;
    const h2 p2 = as_h2((w8 & k.lo) | k.e) - off_lo;
    const h2 p3 = as_h2((w8 & k.hi) | k.e) - off_hi;
    ea = __builtin_amdgcn_fdot2(p0, as_h2(xv.x), ea, false);
    eb = __builtin_amdgcn_fdot2(p1, as_h2(xv.y), eb, false);
    ea = __builtin_amdgcn_fdot2(p2, as_h2(xv.z), ea, false);
    eb = __builtin_amdgcn_fdot2(p3, as_h2(xv.w), eb, false);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Wave-wide sum with DPP moves inside each 16-lane row (xor 1, xor 2, half
// mirror, mirror) and four lane reads for the rows; the result is uniform.
#define AW4_DPP_ADD(v, ctrl)                                                                        \
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, \
                                                               0xF, 0xF, true))
__device__ __forceinline__ float wave_sum_fast(float v) {
    AW4_DPP_ADD(v, 0xB1);    // quad_perm [1,0,3,2]
    AW4_DPP_ADD(v, 0x4E);    // quad_perm [2,3,0,1]
    AW4_DPP_ADD(v, 0x141);   // row_half_mirror
    AW4_DPP_ADD(v, 0x140);   // row_mirror
    const int iv = __builtin_bit_cast(int, v);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 0)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 16)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 32)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 48));
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

// logistic function with the hardware reciprocal (about 1 ulp, like __expf)
__device__ __forceinline__ float sigmoidf_(float v) { return __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }

// block-wide sum over 256 threads; red must hold 4 floats
__device__ __forceinline__ float block_sum256(float v, float* red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

template <int PRO>
__device__ void gemv_prologue(const GemvArgs& a, _Float16* xs, float* red) {
    const int K = a.K;
    if (PRO == PRO_NORM) {
        float ss = 0.f;
        for (int k = threadIdx.x; k < K; k += 256) {
            float v = a.x[k];
            ss += v * v;
        }
        ss = block_sum256(ss, red);
        const float r = 1.0f / sqrtf(ss / (float)K + a.eps);
        for (int k = threadIdx.x; k < K; k += 256) xs[k] = (_Float16)(a.x[k] * r * a.nw[k]);
    } else if (PRO == PRO_GATED) {
        // per head of gated_d values: RMSNorm(o) * w * SiLU(z)
        const int d = a.gated_d, nh = K / d;
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        for (int hh = wave; hh < nh; hh += 4) {
            const float* o = a.x + (int64_t)hh * d;
            float ss = 0.f;
            for (int i = lane; i < d; i += 64) ss += o[i] * o[i];
            ss = wave_sum(ss);
            const float r = 1.0f / sqrtf(ss / (float)d + a.eps);
            for (int i = lane; i < d; i += 64) {
                float zz = a.z[(int64_t)hh * d + i];
                float silu = zz * sigmoidf_(zz);
                xs[hh * d + i] = (_Float16)(o[i] * r * a.nw[i] * silu);
            }
        }
    } else {
        for (int k = threadIdx.x; k < K; k += 256) xs[k] = a.h[k];
    }
}

template <int PRO, int EPI>
__global__ __launch_bounds__(256) void k_gemv_w4(GemvArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    float* red = (float*)smem;
    _Float16* xs = (_Float16*)(smem + 64);
    gemv_prologue<PRO>(a, xs, red);
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int K = a.K;
    const int nchunk = K >> 4;
    const int64_t dw_row = K >> 3;
    const int g_row = K >> 5;
    const int npairs = (a.rows + 1) >> 1;
    const uint4* xv = (const uint4*)xs;   // 8 halves per uint4, chunk c -> xv[2c], xv[2c+1]
    for (int pr = blockIdx.x * 4 + wave; pr < npairs; pr += gridDim.x * 4) {
        const int r0 = pr * 2;
        const bool has1 = (r0 + 1) < a.rows;
        const int r1 = has1 ? r0 + 1 : r0;
        const uint2* c0 = (const uint2*)(a.codes + (int64_t)r0 * dw_row);
        const uint2* c1 = (const uint2*)(a.codes + (int64_t)r1 * dw_row);
        const uint16_t* s0 = a.scales + (int64_t)r0 * g_row;
        const uint16_t* s1 = a.scales + (int64_t)r1 * g_row;
        float acc0 = 0.f, acc1 = 0.f;
        for (int c = lane; c < nchunk; c += 64) {
            const uint2 w0 = c0[c];
            const uint2 w1 = c1[c];
            const float sc0 = half_bits_to_float(s0[c >> 1]);
            const float sc1 = half_bits_to_float(s1[c >> 1]);
            const uint4 xa = xv[2 * c], xb = xv[2 * c + 1];
            float a0 = 0.f, b0 = 0.f, a1 = 0.f, b1 = 0.f;
            dq_dot8(w0.x, xa, a0, b0);
            dq_dot8(w0.y, xb, a0, b0);
            dq_dot8(w1.x, xa, a1, b1);
            dq_dot8(w1.y, xb, a1, b1);
            acc0 += sc0 * (a0 + 0.0625f * b0);
            acc1 += sc1 * (a1 + 0.0625f * b1);
        }
        acc0 = wave_sum(acc0);
        acc1 = wave_sum(acc1);
        if (lane == 0) {
            if (EPI == EPI_STORE) {
                a.y[r0] = acc0;
                if (has1) a.y[r0 + 1] = acc1;
            } else if (EPI == EPI_RESID) {
                a.y[r0] += acc0;
                if (has1) a.y[r0 + 1] += acc1;
            } else {
                // interleaved pair: row 2i is gate i, row 2i+1 is up i
                const float g = acc0;
                a.hout[pr] = (_Float16)(g * sigmoidf_(g) * acc1);
            }
        }
    }
}

// ------------------------------------------------------------------ compile-time prologues
// Two phases: load() issues every load of the prologue at once (vector loads,
// fully unrolled) and must run before the kernel issues its weight loads, so
// that the short L2 reads of the input vector are not queued behind the HBM
// reads of the codes (vector memory counters retire in issue order);
// finish() reduces and writes the fp16 input vector to LDS.
// LDS image of the fp16 input.  Flat: element k at k.  Padded: each 32-value
// group g at 40 g halves (80 bytes), so that lanes reading consecutive groups
// with 16-byte LDS reads start on different banks (a 64-byte lane stride puts
// every other lane on the same banks).
template <bool PAD>
__host__ __device__ constexpr int xs_at(int k) { return PAD ? (k >> 5) * 40 + (k & 31) : k; }
template <bool PAD>
__host__ __device__ constexpr int xs_len(int K) { return PAD ? (K >> 5) * 40 : K; }

template <int K, int PRO, bool PAD = false>
struct Prologue;

template <int K, bool PAD>
struct Prologue<K, PRO_NORM, PAD> {
    static constexpr int N4 = K / 4;
    static constexpr int PER = (N4 + 255) / 256;
    float4 v[PER], w[PER];
    __device__ __forceinline__ void load(const GemvArgs& a) {
        const float4* x4 = (const float4*)a.x;
        const float4* w4 = (const float4*)a.nw;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = threadIdx.x + 256 * i;
            if (N4 % 256 == 0 || idx < N4) {
                v[i] = x4[idx];
                w[i] = w4[idx];
            } else {
                v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
                w[i] = v[i];
            }
        }
    }
    __device__ __forceinline__ void finish(const GemvArgs& a, _Float16* xs, float* red) {
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i) ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
        ss = wave_sum_fast(ss);
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) red[wave] = ss;
        __syncthreads();
        ss = red[0] + red[1] + red[2] + red[3];
        const float r = 1.0f / sqrtf(ss / (float)K + a.eps);
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = threadIdx.x + 256 * i;
            if (N4 % 256 == 0 || idx < N4) {
                h4 o = {(_Float16)(v[i].x * r * w[i].x), (_Float16)(v[i].y * r * w[i].y),
                        (_Float16)(v[i].z * r * w[i].z), (_Float16)(v[i].w * r * w[i].w)};
                *(h4*)(xs + xs_at<PAD>(4 * idx)) = o;
            }
        }
    }
};

// gated RMSNorm per head of d values: RMSNorm(o) * w * SiLU(z).  Thread t
// takes E = K/256 consecutive values; the d/E threads of a head reduce with
// lane shuffles.
template <int K, bool PAD>
struct Prologue<K, PRO_GATED, PAD> {
    static constexpr int E = K >= 256 ? K / 256 : 1;
    static constexpr int V4 = E % 4 == 0 ? E / 4 : 0;   // float4 loads per array when E allows
    float ov[E], zv[E], wv[E];
    __device__ __forceinline__ void load(const GemvArgs& a) {
        const int base = threadIdx.x * E;
        const bool live = base < K;   // K < 256: threads past K idle (whole waves)
        const int c0 = live ? base % a.gated_d : 0;
        if (V4) {
#pragma unroll
            for (int i = 0; i < V4; ++i) {
                const float4 o = ((const float4*)(a.x + base))[i];
                const float4 z = ((const float4*)(a.z + base))[i];
                const float4 w = ((const float4*)(a.nw + c0))[i];
                ov[4 * i] = o.x; ov[4 * i + 1] = o.y; ov[4 * i + 2] = o.z; ov[4 * i + 3] = o.w;
                zv[4 * i] = z.x; zv[4 * i + 1] = z.y; zv[4 * i + 2] = z.z; zv[4 * i + 3] = z.w;
                wv[4 * i] = w.x; wv[4 * i + 1] = w.y; wv[4 * i + 2] = w.z; wv[4 * i + 3] = w.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                ov[e] = live ? a.x[base + e] : 0.f;
                zv[e] = live ? a.z[base + e] : 0.f;
                wv[e] = live ? a.nw[c0 + e] : 0.f;
            }
        }
    }
    __device__ __forceinline__ void finish(const GemvArgs& a, _Float16* xs, float*) {
        const int base = threadIdx.x * E;
        const int d = a.gated_d;
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) ss += ov[e] * ov[e];
        const int tph = d / E;   // threads per head (power of two, <= 64)
        for (int m = tph >> 1; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
        const float r = 1.0f / sqrtf(ss / (float)d + a.eps);
        if (base < K) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float silu = zv[e] * sigmoidf_(zv[e]);
                xs[xs_at<PAD>(base + e)] = (_Float16)(ov[e] * r * wv[e] * silu);
            }
        }
    }
};

template <int K, bool PAD>
struct Prologue<K, PRO_LOADH, PAD> {
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    static constexpr int N8 = K / 8;
    static constexpr int PER = (N8 + 255) / 256;
    v4u v[PER];
    __device__ __forceinline__ void load(const GemvArgs& a) {
        const v4u* src = (const v4u*)a.h;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = threadIdx.x + 256 * i;
            v[i] = src[idx < N8 ? idx : N8 - 1];   // clamped: straight-line loads, stores guarded
        }
        // pin every load here: otherwise the compiler sinks the loads of a
        // partial last slice into the guarded stores, one branch and one full
        // memory wait each (four serial cache round trips at K = 17408)
#pragma unroll
        for (int i = 0; i < PER; ++i) asm volatile("" : "+v"(v[i]));
    }
    __device__ __forceinline__ void finish(const GemvArgs&, _Float16* xs, float*) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = threadIdx.x + 256 * i;
            if (N8 % 256 == 0 || idx < N8) *(v4u*)(xs + xs_at<PAD>(8 * idx)) = v[i];
        }
    }
};

// ------------------------------------------------------------------ streaming W4 GEMV
// Specialised for a compile-time row length K = 32 G.  A wave owns a block of
// R consecutive rows (R G a multiple of 64, R >= 2) which are contiguous in
// memory; lane l takes the NF = R G / 64 groups f = l + 64 i (row f / G, group
// f % G), one 16-byte load of 32 codes and one fp16 scale each, so every wave
// load covers 1 KB of contiguous codes and every lane does the same work.
// The loads of the wave's first row block are issued before the prologue and
// those of the next block before the current one is reduced, so HBM streaming
// overlaps the input normalisation and the cross-lane reductions.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kStreamMaxPer = 10;   // row blocks per wave the pipelined path unrolls

// Two forms of the streaming kernel.  The 27B-shape projections (K = 4096,
// 5120, 6144: NF = 4, 5, 6) read the input slices from LDS at each use and keep
// one row block in registers per wave (55-80 VGPRs), so that 4 (NF 4, 6) or 6
// (NF 5) waves share a SIMD and the wave count, not a deep per-wave pipeline,
// keeps the loads in flight: measured faster than the register-resident form
// (2 waves per SIMD, x in registers, a three-deep ring of row blocks) by 2% of
// a decode step.  Other row lengths keep the register-resident form.
__host__ __device__ constexpr bool stream_lds_x(int NF) { return NF == 4 || NF == 5 || NF == 6; }
__host__ __device__ constexpr int stream_simd_waves(int NF) { return NF == 5 ? 6 : stream_lds_x(NF) ? 4 : 2; }

template <int R, int NF>
struct RowBlock {
    u32x4 c[NF];
    uint16_t s[NF];
};

template <int R, int NF>
__device__ __forceinline__ void load_block(RowBlock<R, NF>& b, const uint32_t* __restrict__ codes,
                                           const uint16_t* __restrict__ scales, int rb, int G, int lane) {
    const u32x4* cb = (const u32x4*)(codes + (int64_t)rb * R * G * 4);
    const uint16_t* sb = scales + (int64_t)rb * R * G;
#pragma unroll
    for (int i = 0; i < NF; ++i) {
        b.c[i] = __builtin_nontemporal_load(cb + lane + 64 * i);
        b.s[i] = sb[lane + 64 * i];
    }
}

template <int R, int NF, int PRO, int EPI>
__global__ __launch_bounds__(256, stream_simd_waves(NF)) void k_gemv_stream(GemvArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    float* red = (float*)smem;
    _Float16* xs = (_Float16*)(smem + 64);
    constexpr int G = 64 * NF / R;
    // pipeline the codes across row blocks only while the buffers stay small
    constexpr bool kPipe = NF <= 8 && !stream_lds_x(NF);
    constexpr bool kXreg = kPipe;   // the input slices stay in registers
    constexpr int kDepth = 3;
    constexpr int kMaxPer = kStreamMaxPer;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nrb = a.rows / R;
    const int nw = gridDim.x * 4;
    int rb = blockIdx.x * 4 + wave;

    // The input vector first, then the weights: issued together, the input's
    // short cache reads queue behind the chip-wide flood of weight requests
    // and every block waits several microseconds for its prologue.
    Prologue<32 * G, PRO, true> pro;
    pro.load(a);
    pro.finish(a, xs, red);
    __syncthreads();
    RowBlock<R, NF> ring[kPipe ? kDepth : 1];   // ring[0]: the wave's first block
    if (rb < nrb) load_block<R, NF>(ring[0], a.codes, a.scales, rb, G, lane);
    // residual epilogue: the wave's old values, loaded ahead (lane r holds row
    // r) so the epilogue is a plain store instead of a dependent read-modify-write
    float yold = 0.f;
    if (EPI == EPI_RESID && rb < nrb && lane < R) yold = a.y[rb * R + lane];

    int row_of[NF], grp_of[NF];
#pragma unroll
    for (int i = 0; i < NF; ++i) {
        const int f = lane + 64 * i;
        row_of[i] = f / G;
        grp_of[i] = f % G;
    }
    const uint4* xv = (const uint4*)xs;   // group g: xv[5g .. 5g+3] (padded image)
    // short rows: this lane's slices of the input stay in registers for every
    // row block (the lane -> group map is the same for all of them)
    uint4 xr[kXreg ? NF : 1][4];
    if (kXreg) {
#pragma unroll
        for (int i = 0; i < NF; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k) xr[kXreg ? i : 0][k] = xv[5 * grp_of[i] + k];
    }
    const NibK nk;

    // dot products of one row block and the epilogue (yo: the lane's old
    // residual value, lane r holding row r)
    auto body = [&](const RowBlock<R, NF>& b, int rbb, float yo) {
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll
        for (int i = 0; i < NF; ++i) {
            uint4 x0, x1, x2, x3;
            if (kXreg) {
                x0 = xr[kXreg ? i : 0][0]; x1 = xr[kXreg ? i : 0][1];
                x2 = xr[kXreg ? i : 0][2]; x3 = xr[kXreg ? i : 0][3];
            } else {
                const int g = grp_of[i];
                x0 = xv[5 * g]; x1 = xv[5 * g + 1]; x2 = xv[5 * g + 2]; x3 = xv[5 * g + 3];
            }
            float ea = 0.f, eb = 0.f;
            dq_dot8(b.c[i][0], x0, ea, eb, nk);
            dq_dot8(b.c[i][1], x1, ea, eb, nk);
            dq_dot8(b.c[i][2], x2, ea, eb, nk);
            dq_dot8(b.c[i][3], x3, ea, eb, nk);
            const float part = half_bits_to_float(b.s[i]) * (ea + 0.0625f * eb);
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] += row_of[i] == r ? part : 0.f;
            // long rows: split the group loop in two so that the compiler hoists
            // at most half of the LDS reads (16 registers per group)
            if (!kXreg && i == NF / 2) asm volatile("" ::: "memory");
        }
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = wave_sum_fast(acc[r]);
        const int r0 = rbb * R;
        if (EPI == EPI_RESID) {
            // lane r adds row r's dot product (acc is uniform across the wave)
            float mine = 0.f;
#pragma unroll
            for (int r = 0; r < R; ++r) mine = lane == r ? acc[r] : mine;
            if (lane < R) a.y[r0 + lane] = yo + mine;
        } else if (lane == 0) {
            if (EPI == EPI_STORE) {
#pragma unroll
                for (int r = 0; r < R; ++r) a.y[r0 + r] = acc[r];
            } else {
#pragma unroll
                for (int r = 0; r < R; r += 2) {
                    const float g = acc[r];
                    a.hout[(r0 + r) >> 1] = (_Float16)(g * sigmoidf_(g) * acc[r + 1]);
                }
            }
        }
    };

    if (rb >= nrb) return;
    if (kPipe) {
        // a ring of PD register sets, each filled PD - 1 row blocks ahead of its
        // use (fully unrolled: no copies between sets); every step issues the
        // same loads, so no wait ever drains the ring
        constexpr int PD = kDepth;
        float yr[PD];
        // a prefetch past the wave's last block reads block 0 instead: one
        // small region every such wave shares, so it stays in L2 and costs no
        // HBM traffic (the data is never used)
        yr[0] = yold;
#pragma unroll
        for (int k = 1; k < PD - 1; ++k) {
            const int bk = rb + k * nw < nrb ? rb + k * nw : 0;
            load_block<R, NF>(ring[k], a.codes, a.scales, bk, G, lane);
            if (EPI == EPI_RESID && lane < R) yr[k] = a.y[bk * R + lane];
        }
        // straight-line steps (no loop header, so the wait counts stay exact);
        // the launch keeps every wave within kMaxPer blocks, the tail loop
        // below only keeps other launches correct
#pragma unroll
        for (int j = 0; j < kMaxPer; ++j) {
            const int bl = rb + (j + PD - 1) * nw < nrb ? rb + (j + PD - 1) * nw : 0;
            load_block<R, NF>(ring[(j + PD - 1) % PD], a.codes, a.scales, bl, G, lane);
            if (EPI == EPI_RESID && lane < R) yr[(j + PD - 1) % PD] = a.y[bl * R + lane];
            asm volatile("" ::: "memory");   // issue the prefetch before this block's math
            body(ring[j % PD], rb + j * nw, yr[j % PD]);
            if (rb + (j + 1) * nw >= nrb) break;
        }
        for (int rx = rb + kMaxPer * nw; rx < nrb; rx += nw) {
            load_block<R, NF>(ring[0], a.codes, a.scales, rx, G, lane);
            body(ring[0], rx, EPI == EPI_RESID && lane < R ? a.y[rx * R + lane] : 0.f);
        }
    } else {
        for (; rb < nrb; rb += nw) {
            body(ring[0], rb, yold);
            if (rb + nw < nrb) {
                load_block<R, NF>(ring[0], a.codes, a.scales, rb + nw, G, lane);
                if (EPI == EPI_RESID && lane < R) yold = a.y[(rb + nw) * R + lane];
            }
        }
    }
}

// ------------------------------------------------------------------ int8 output head
// int8 pair -> exact fp16 pair: flip to offset binary b = c + 128, place each
// byte under exponent byte 0x64 (fp16 1024 + b) and subtract 1152.
__device__ __forceinline__ void i8_dot4(uint32_t w, uint32_t x01, uint32_t x23, float& acc) {
    const h2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t b = w ^ 0x80808080u;
    const h2 p01 = as_h2(__builtin_amdgcn_perm(0x64646464u, b, 0x04010400u)) - off;
    const h2 p23 = as_h2(__builtin_amdgcn_perm(0x64646464u, b, 0x04030402u)) - off;
    acc = __builtin_amdgcn_fdot2(p01, as_h2(x01), acc, false);
    acc = __builtin_amdgcn_fdot2(p23, as_h2(x23), acc, false);
}

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

__global__ __launch_bounds__(256) void k_head_i8(HeadArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    float* red = (float*)smem;
    _Float16* xs = (_Float16*)(smem + 64);
    __shared__ float bv_s[4];
    __shared__ int bi_s[4];
    {
        GemvArgs g{};
        g.K = a.H;
        g.x = a.x;
        g.nw = a.nw;
        g.eps = a.eps;
        gemv_prologue<PRO_NORM>(g, xs, red);
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H = a.H;
    const int nchunk = H >> 4;    // 16 int8 per chunk (one uint4)
    const int g_row = H >> 5;
    const int npairs = (a.V + 1) >> 1;
    const uint4* xv = (const uint4*)xs;
    float best = -INFINITY;
    int besti = 0x7fffffff;
    for (int pr = blockIdx.x * 4 + wave; pr < npairs; pr += gridDim.x * 4) {
        const int r0 = pr * 2;
        const bool has1 = (r0 + 1) < a.V;
        const int r1 = has1 ? r0 + 1 : r0;
        const int64_t q0 = a.map ? a.map[r0] : r0, q1 = a.map ? a.map[r1] : r1;
        const uint4* c0 = (const uint4*)(a.codes + q0 * H);
        const uint4* c1 = (const uint4*)(a.codes + q1 * H);
        const uint16_t* s0 = a.scales + q0 * g_row;
        const uint16_t* s1 = a.scales + q1 * g_row;
        float acc0 = 0.f, acc1 = 0.f;
        for (int c = lane; c < nchunk; c += 64) {
            const uint4 w0 = c0[c], w1 = c1[c];
            const float sc0 = half_bits_to_float(s0[c >> 1]);
            const float sc1 = half_bits_to_float(s1[c >> 1]);
            const uint4 xa = xv[2 * c], xb = xv[2 * c + 1];
            float p0 = 0.f, p1 = 0.f;
            i8_dot4(w0.x, xa.x, xa.y, p0);
            i8_dot4(w0.y, xa.z, xa.w, p0);
            i8_dot4(w0.z, xb.x, xb.y, p0);
            i8_dot4(w0.w, xb.z, xb.w, p0);
            i8_dot4(w1.x, xa.x, xa.y, p1);
            i8_dot4(w1.y, xa.z, xa.w, p1);
            i8_dot4(w1.z, xb.x, xb.y, p1);
            i8_dot4(w1.w, xb.z, xb.w, p1);
            acc0 += sc0 * p0;
            acc1 += sc1 * p1;
        }
        acc0 = wave_sum(acc0);
        acc1 = wave_sum(acc1);
        if (lane == 0 && a.logits) {
            a.logits[r0] = acc0;
            if (has1) a.logits[r0 + 1] = acc1;
        }
        if (better(acc0, r0, best, besti)) { best = acc0; besti = r0; }
        if (has1 && better(acc1, r0 + 1, best, besti)) { best = acc1; besti = r0 + 1; }
    }
    if (lane == 0) {
        bv_s[wave] = best;
        bi_s[wave] = besti;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float b = bv_s[0];
        int bi = bi_s[0];
        for (int w = 1; w < 4; ++w)
            if (better(bv_s[w], bi_s[w], b, bi)) { b = bv_s[w]; bi = bi_s[w]; }
        a.part_val[blockIdx.x] = b;
        a.part_idx[blockIdx.x] = bi;
    }
}

// Streaming int8 head for rows of H = 1024 k bytes: lane l takes the NC = H/1024
// 16-byte chunks l + 64 i of every row (one 1 KB wave load per chunk index),
// keeps its slices of the normalised input in registers, and streams rows
// through a ring of three register sets filled two rows ahead.  The loop is
// unrolled by three with the same loads in flight at its entry and at its
// back edge, so the compiler's wait counts stay exact; a prefetch past the
// wave's last row reads row 0 instead (an L2 hit, the data is never used).
// MAPPED: output i reads table row map[i] (the draft head's id list); the id is
// fetched with a scalar load, whose wait does not drain the ring's vector loads.
template <int H, bool MAPPED>
__global__ __launch_bounds__(256, 2) void k_head_stream(HeadArgs a) {
    constexpr int NC = H / 1024;
    constexpr int GR = H / 32;
    extern __shared__ __align__(16) unsigned char smem[];
    float* red = (float*)smem;
    _Float16* xs = (_Float16*)(smem + 64);
    __shared__ float bv_s[4];
    __shared__ int bi_s[4];
    {
        GemvArgs g{};
        g.K = H;
        g.x = a.x;
        g.nw = a.nw;
        g.eps = a.eps;
        Prologue<H, PRO_NORM> pro;
        pro.load(g);
        pro.finish(g, xs, red);
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nw = gridDim.x * 4;
    const int r0 = blockIdx.x * 4 + wave;
    const uint4* xv = (const uint4*)xs;
    uint4 xa[NC], xb[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        xa[i] = xv[2 * (lane + 64 * i)];
        xb[i] = xv[2 * (lane + 64 * i) + 1];
    }
    struct Row {
        u32x4 c[NC];
        uint16_t s[NC];
    };
    auto load = [&](Row& b, int row) {
        const int64_t src = MAPPED ? (int64_t)a.map[__builtin_amdgcn_readfirstlane(row)] : row;
        const u32x4* cp = (const u32x4*)(a.codes + src * H);
        const uint16_t* sp = a.scales + src * GR;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            b.c[i] = __builtin_nontemporal_load(cp + lane + 64 * i);
            b.s[i] = sp[(lane + 64 * i) >> 1];
        }
    };
    float best = -INFINITY;
    int besti = 0x7fffffff;
    auto body = [&](const Row& b, int row) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            float p = 0.f;
            i8_dot4(b.c[i][0], xa[i].x, xa[i].y, p);
            i8_dot4(b.c[i][1], xa[i].z, xa[i].w, p);
            i8_dot4(b.c[i][2], xb[i].x, xb[i].y, p);
            i8_dot4(b.c[i][3], xb[i].z, xb[i].w, p);
            acc += half_bits_to_float(b.s[i]) * p;
        }
        acc = wave_sum_fast(acc);
        if (lane == 0 && a.logits) a.logits[row] = acc;
        if (better(acc, row, best, besti)) { best = acc; besti = row; }
    };
    if (r0 < a.V) {
        Row ring[3];
        auto clampr = [&](int row) { return row < a.V ? row : 0; };
        load(ring[0], r0);
        load(ring[1], clampr(r0 + nw));
        for (int row = r0;; row += 3 * nw) {
            load(ring[2], clampr(row + 2 * nw));
            asm volatile("" ::: "memory");
            body(ring[0], row);
            if (row + nw >= a.V) break;
            load(ring[0], clampr(row + 3 * nw));
            asm volatile("" ::: "memory");
            body(ring[1], row + nw);
            if (row + 2 * nw >= a.V) break;
            load(ring[1], clampr(row + 4 * nw));
            asm volatile("" ::: "memory");
            body(ring[2], row + 2 * nw);
            if (row + 3 * nw >= a.V) break;
        }
    }
    if (lane == 0) {
        bv_s[wave] = best;
        bi_s[wave] = besti;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float b = bv_s[0];
        int bi = bi_s[0];
        for (int w = 1; w < 4; ++w)
            if (better(bv_s[w], bi_s[w], b, bi)) { b = bv_s[w]; bi = bi_s[w]; }
        a.part_val[blockIdx.x] = b;
        a.part_idx[blockIdx.x] = bi;
    }
}

// ------------------------------------------------------------------ M-vector W4 GEMV
// The verify pass of draft tokens runs M <= 4 tokens through every layer in
// one sweep over the weights: each group of codes is loaded and dequantised
// once and dotted with the M input vectors held in LDS.
// LDS image of the M input vectors: flat [M][K], or with each 32-value group
// padded to 40 halves (80 bytes), so that lanes reading consecutive groups hit
// distinct banks
template <bool PAD>
__device__ __forceinline__ int xs_index(int k) { return PAD ? (k >> 5) * 40 + (k & 31) : k; }
template <bool PAD>
__device__ __forceinline__ int xs_stride(int K) { return PAD ? (K >> 5) * 40 : K; }

template <int MAXM, bool PAD = false>
__device__ __forceinline__ void multi_prologue(int pro, const GemvMultiArgs& a, _Float16* xs, float* red) {
    const int K = a.K, M = a.M, KP = xs_stride<PAD>(K);
    if (pro == PRO_LOADH) {
        for (int m = 0; m < M; ++m) {
            const uint4* src = (const uint4*)(a.h + m * a.sh);
            for (int i = threadIdx.x; i < K / 8; i += 256) *(uint4*)(xs + m * KP + xs_index<PAD>(8 * i)) = src[i];
        }
        return;
    }
    if (pro == PRO_NORM) {
        float ss[MAXM];
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            ss[m] = 0.f;
            if (m < M)
                for (int k = threadIdx.x; k < K; k += 256) {
                    const float v = a.x[m * a.sx + k];
                    ss[m] += v * v;
                }
            ss[m] = wave_sum(ss[m]);
        }
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        if (lane == 0)
#pragma unroll
            for (int m = 0; m < MAXM; ++m) red[m * 4 + wave] = ss[m];
        __syncthreads();
        for (int m = 0; m < M; ++m) {
            const float t = red[m * 4] + red[m * 4 + 1] + red[m * 4 + 2] + red[m * 4 + 3];
            const float r = 1.0f / sqrtf(t / (float)K + a.eps);
            for (int k = threadIdx.x; k < K; k += 256)
                xs[m * KP + xs_index<PAD>(k)] = (_Float16)(a.x[m * a.sx + k] * r * a.nw[k]);
        }
        return;
    }
    // gated: per head of d values RMSNorm(o) * w * SiLU(z).  Thread t takes E
    // consecutive values (E = K/256 when that divides a head, as in the
    // single-vector prologue); the d/E threads of a head reduce with shuffles.
    const int d = a.gated_d;
    const int E = K >= 256 && K % 256 == 0 && d % (K / 256) == 0 && d / (K / 256) <= 64 ? K / 256 : 0;
    if (E == 16) {
        const int base = threadIdx.x * 16, c0 = base % d;
        float wv[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 w = ((const float4*)(a.nw + c0))[i];
            wv[4 * i] = w.x; wv[4 * i + 1] = w.y; wv[4 * i + 2] = w.z; wv[4 * i + 3] = w.w;
        }
        const int tph = d / 16;
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            if (m < M) {
                float ov[16], zv[16];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float4 o = ((const float4*)(a.x + m * a.sx + base))[i];
                    const float4 z = ((const float4*)(a.z + m * a.sz + base))[i];
                    ov[4 * i] = o.x; ov[4 * i + 1] = o.y; ov[4 * i + 2] = o.z; ov[4 * i + 3] = o.w;
                    zv[4 * i] = z.x; zv[4 * i + 1] = z.y; zv[4 * i + 2] = z.z; zv[4 * i + 3] = z.w;
                }
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 16; ++e) ss += ov[e] * ov[e];
                for (int mm = tph >> 1; mm >= 1; mm >>= 1) ss += __shfl_xor(ss, mm, 64);
                const float r = 1.0f / sqrtf(ss / (float)d + a.eps);
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    xs[m * KP + xs_index<PAD>(base + e)] = (_Float16)(ov[e] * r * wv[e] * (zv[e] * sigmoidf_(zv[e])));
            }
        }
        return;
    }
    // other shapes: one wave per head
    const int nh = K / d;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int m = 0; m < M; ++m)
        for (int hh = wave; hh < nh; hh += 4) {
            const float* o = a.x + m * a.sx + (int64_t)hh * d;
            const float* z = a.z + m * a.sz + (int64_t)hh * d;
            float ss = 0.f;
            for (int i = lane; i < d; i += 64) ss += o[i] * o[i];
            ss = wave_sum(ss);
            const float r = 1.0f / sqrtf(ss / (float)d + a.eps);
            for (int i = lane; i < d; i += 64)
                xs[m * KP + xs_index<PAD>(hh * d + i)] = (_Float16)(o[i] * r * a.nw[i] * (z[i] * sigmoidf_(z[i])));
        }
}

template <int R, int NF, int PRO, int EPI>
__global__ __launch_bounds__(256, 2) void k_gemv_multi(GemvMultiArgs a) {
    constexpr int MAXM = 4;
    extern __shared__ __align__(16) unsigned char smem[];
    float* red = (float*)smem;                       // 16 floats
    _Float16* xs = (_Float16*)(smem + 64);           // [M][KP]
    constexpr int G = 64 * NF / R;
    constexpr int K = 32 * G;
    constexpr bool kPad = NF <= 8;                   // padded image fits LDS for M = 4
    constexpr int KP = kPad ? G * 40 : K;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nrb = (a.rows + R - 1) / R;            // the last row block may be partial
    const int nw = gridDim.x * 4;
    const int M = a.M;
    int row_of[NF], grp_of[NF];
#pragma unroll
    for (int i = 0; i < NF; ++i) {
        const int f = lane + 64 * i;
        row_of[i] = f / G;
        grp_of[i] = f % G;
    }
    auto load = [&](RowBlock<R, NF>& b, int rbk) {
        const u32x4* cb = (const u32x4*)(a.codes + (int64_t)rbk * R * G * 4);
        const uint16_t* sb = a.scales + (int64_t)rbk * R * G;
#pragma unroll
        for (int i = 0; i < NF; ++i) {
            if (rbk * R + row_of[i] < a.rows) {
                b.c[i] = __builtin_nontemporal_load(cb + lane + 64 * i);
                b.s[i] = sb[lane + 64 * i];
            } else {
                b.c[i] = u32x4{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
                b.s[i] = 0;
            }
        }
    };
    // the input vectors first (see k_gemv_stream), then the weights
    multi_prologue<MAXM, kPad>(PRO, a, xs, red);
    __syncthreads();
    int rb = blockIdx.x * 4 + wave;
    if (rb >= nrb) return;
    RowBlock<R, NF> cur;
    load(cur, rb);
    const NibK nk;
    const h2 off_lo = {(_Float16)1032.0f, (_Float16)1032.0f};
    const h2 off_hi = {(_Float16)1152.0f, (_Float16)1152.0f};

    // one row block: each code dword is dequantised once and dotted with the
    // M inputs (read from LDS)
    auto body = [&](const RowBlock<R, NF>& b, int rbb) {
        float acc[MAXM][R];
#pragma unroll
        for (int m = 0; m < MAXM; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r) acc[m][r] = 0.f;
#pragma unroll
        for (int i = 0; i < NF; ++i) {
            const int g = grp_of[i];
            const float sc = half_bits_to_float(b.s[i]);
            h2 p[4][4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t w = b.c[i][d], w8 = w >> 8;
                p[d][0] = as_h2((w & nk.lo) | nk.e) - off_lo;
                p[d][1] = as_h2((w & nk.hi) | nk.e) - off_hi;
                p[d][2] = as_h2((w8 & nk.lo) | nk.e) - off_lo;
                p[d][3] = as_h2((w8 & nk.hi) | nk.e) - off_hi;
            }
#pragma unroll
            for (int m = 0; m < MAXM; ++m) {
                if (m < M) {
                    const uint4* xv = (const uint4*)(xs + m * KP + (kPad ? 40 : 32) * g);
                    float ea = 0.f, eb = 0.f;
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const uint4 x = xv[d];
                        ea = __builtin_amdgcn_fdot2(p[d][0], as_h2(x.x), ea, false);
                        eb = __builtin_amdgcn_fdot2(p[d][1], as_h2(x.y), eb, false);
                        ea = __builtin_amdgcn_fdot2(p[d][2], as_h2(x.z), ea, false);
                        eb = __builtin_amdgcn_fdot2(p[d][3], as_h2(x.w), eb, false);
                    }
                    const float part = sc * (ea + 0.0625f * eb);
#pragma unroll
                    for (int r = 0; r < R; ++r) acc[m][r] += row_of[i] == r ? part : 0.f;
                }
            }
            if (NF > 8 && i == NF / 2) asm volatile("" ::: "memory");
        }
        const int r0 = rbb * R;
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            if (m < M) {
#pragma unroll
                for (int r = 0; r < R; ++r) acc[m][r] = wave_sum_fast(acc[m][r]);
                if (lane == 0) {
                    if (EPI == EPI_STORE) {
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            if (r0 + r < a.rows) a.y[m * a.sy + r0 + r] = acc[m][r];
                    } else if (EPI == EPI_RESID) {
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            if (r0 + r < a.rows) a.y[m * a.sy + r0 + r] += acc[m][r];
                    } else {
#pragma unroll
                        for (int r = 0; r < R; r += 2) {
                            if (r0 + r + 1 < a.rows) {
                                const float gg = acc[m][r];
                                a.hout[m * a.so + ((r0 + r) >> 1)] = (_Float16)(gg * sigmoidf_(gg) * acc[m][r + 1]);
                            }
                        }
                    }
                }
            }
        }
    };

    // at M = 4 the LDS reads of the inputs bound this kernel, not HBM: a plain
    // loop with the next block's loads issued before the epilogue
    for (; rb < nrb; rb += nw) {
        body(cur, rb);
        if (rb + nw < nrb) load(cur, rb + nw);
    }
}

// ------------------------------------------------------------------ multi-input W4 GEMM on MFMA
// M <= 4 input vectors against one W4 matrix on the matrix cores.  A block of
// 16 rows takes one v_mfma_f32_16x16x32_f16 per 32-value group: the A operand
// holds the 16 rows' exact codes (lane (r, q): row r, values 8q..8q+7 of the
// group, i.e. one code dword), the B operand the inputs as columns (lane
// (m, q): input m, the same 8 values, from LDS), so lane (m, q) of the result
// holds the group's unscaled dot products of rows 4q..4q+3 with input m; the
// fp16 group scale is then applied row by row with a mixed-precision FMA.
// Products are exact (small integers times fp16) and accumulate in fp32, as in
// the single-vector kernel.  KS waves of a workgroup share one row block and
// split its groups, adding their partial sums through LDS.  Loads run two
// stages of kStage groups ahead in a ring of three register sets.
constexpr int kStage = 8;

// The M input vectors as fp16 [M][K] in LDS for a compile-time K: every load
// of every input is issued before any is used (one memory round trip), and the
// norms need one barrier.  NORM: RMSNorm(x_m) * w.  LOADH: fp16 copy (two
// inputs per round, to bound the registers).  GATED: per head of d values
// RMSNorm(o) * w * SiLU(z), thread t taking E = K/256 consecutive values.
// input m's row of the image starts at m (K + kMfmaPad) halves: the 32-byte
// pad puts the rows of different inputs on different banks for the lanes of a
// 16-lane row that read the same offset of each
constexpr int kMfmaPad = 16;

template <int K, int PRO>
__device__ __forceinline__ void mfma_prologue(const GemvMultiArgs& a, _Float16* xs, float* red) {
    constexpr int MAXM = 4;
    constexpr int LD = K + kMfmaPad;
    const int M = a.M, tid = threadIdx.x;
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    if (PRO == PRO_NORM) {
        constexpr int N4 = K / 4, PER = (N4 + 255) / 256;
        // straight-line loads (a slice past K or an input past M re-reads a
        // valid one and is zeroed afterwards), pinned before the first use so
        // that no load is sunk into a branch with its own full memory wait
        typedef float f4v __attribute__((ext_vector_type(4)));
        f4v v[MAXM][PER], w[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = tid + 256 * i;
            const int ic = N4 % 256 == 0 || idx < N4 ? idx : N4 - 1;
            w[i] = ((const f4v*)a.nw)[ic];
#pragma unroll
            for (int m = 0; m < MAXM; ++m) v[m][i] = ((const f4v*)(a.x + (m < M ? m : 0) * a.sx))[ic];
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            asm volatile("" : "+v"(w[i]));
#pragma unroll
            for (int m = 0; m < MAXM; ++m) asm volatile("" : "+v"(v[m][i]));
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = tid + 256 * i;
            if (N4 % 256 != 0 && idx >= N4) w[i] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < MAXM; ++m)
                if (m >= M || (N4 % 256 != 0 && idx >= N4)) v[m][i] = f4v{0.f, 0.f, 0.f, 0.f};
        }
        float ss[MAXM];
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            ss[m] = 0.f;
#pragma unroll
            for (int i = 0; i < PER; ++i)
                ss[m] += v[m][i].x * v[m][i].x + v[m][i].y * v[m][i].y + v[m][i].z * v[m][i].z + v[m][i].w * v[m][i].w;
            ss[m] = wave_sum_fast(ss[m]);
        }
        const int wave = tid >> 6;
        if ((tid & 63) == 0)
#pragma unroll
            for (int m = 0; m < MAXM; ++m) red[m * 4 + wave] = ss[m];
        __syncthreads();
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            if (m >= M) break;
            const float r = 1.0f / sqrtf((red[m * 4] + red[m * 4 + 1] + red[m * 4 + 2] + red[m * 4 + 3]) / (float)K + a.eps);
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int idx = tid + 256 * i;
                if (N4 % 256 == 0 || idx < N4) {
                    const h4 o = {(_Float16)(v[m][i].x * r * w[i].x), (_Float16)(v[m][i].y * r * w[i].y),
                                  (_Float16)(v[m][i].z * r * w[i].z), (_Float16)(v[m][i].w * r * w[i].w)};
                    ((h4*)(xs + m * LD))[idx] = o;
                }
            }
        }
    } else if (PRO == PRO_LOADH) {
        constexpr int N8 = K / 8, PER = (N8 + 255) / 256;
#pragma unroll
        for (int m0 = 0; m0 < MAXM; m0 += 2) {
            if (m0 >= M) break;
            typedef uint32_t v4u __attribute__((ext_vector_type(4)));
            v4u v[2][PER];
#pragma unroll
            for (int mm = 0; mm < 2; ++mm)
#pragma unroll
                for (int i = 0; i < PER; ++i) {
                    const int idx = tid + 256 * i;
                    const int m = m0 + mm < M ? m0 + mm : m0;
                    v[mm][i] = ((const v4u*)(a.h + m * a.sh))[idx < N8 ? idx : N8 - 1];
                }
            // pinned: no load sunk into the guarded stores (one wait each)
#pragma unroll
            for (int mm = 0; mm < 2; ++mm)
#pragma unroll
                for (int i = 0; i < PER; ++i) asm volatile("" : "+v"(v[mm][i]));
#pragma unroll
            for (int mm = 0; mm < 2; ++mm)
                if (m0 + mm < M)
#pragma unroll
                    for (int i = 0; i < PER; ++i) {
                        const int idx = tid + 256 * i;
                        if (N8 % 256 == 0 || idx < N8) ((v4u*)(xs + (m0 + mm) * LD))[idx] = v[mm][i];
                    }
        }
    } else {
        constexpr int E = K >= 256 ? K / 256 : 1;
        const int base = tid * E;
        const bool live = base < K;
        const int d = a.gated_d, c0 = live ? base % d : 0;
        const int tph = d / E;   // threads per head (power of two, <= 64)
        // 16-byte loads when a thread's values come in fours (the 27B shape)
        constexpr bool V4 = E % 4 == 0;
        float wv[E];
        if (V4) {
#pragma unroll
            for (int i = 0; i < E / 4; ++i) {
                const float4 w = ((const float4*)(a.nw + c0))[i];
                wv[4 * i] = w.x; wv[4 * i + 1] = w.y; wv[4 * i + 2] = w.z; wv[4 * i + 3] = w.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) wv[e] = live ? a.nw[c0 + e] : 0.f;
        }
#pragma unroll
        for (int m0 = 0; m0 < MAXM; m0 += 2) {
            if (m0 >= M) break;
            float ov[2][E], zv[2][E];
#pragma unroll
            for (int mm = 0; mm < 2; ++mm) {
                const int m = m0 + mm < M ? m0 + mm : m0;
                if (V4) {
#pragma unroll
                    for (int i = 0; i < E / 4; ++i) {
                        const float4 o = ((const float4*)(a.x + m * a.sx + base))[i];
                        const float4 z = ((const float4*)(a.z + m * a.sz + base))[i];
                        ov[mm][4 * i] = o.x; ov[mm][4 * i + 1] = o.y; ov[mm][4 * i + 2] = o.z; ov[mm][4 * i + 3] = o.w;
                        zv[mm][4 * i] = z.x; zv[mm][4 * i + 1] = z.y; zv[mm][4 * i + 2] = z.z; zv[mm][4 * i + 3] = z.w;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        ov[mm][e] = live ? a.x[m * a.sx + base + e] : 0.f;
                        zv[mm][e] = live ? a.z[m * a.sz + base + e] : 0.f;
                    }
                }
            }
#pragma unroll
            for (int mm = 0; mm < 2; ++mm) {
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) ss += ov[mm][e] * ov[mm][e];
                for (int o = tph >> 1; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
                const float r = 1.0f / sqrtf(ss / (float)d + a.eps);
                if (live && m0 + mm < M)
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        xs[(m0 + mm) * LD + base + e] =
                            (_Float16)(ov[mm][e] * r * wv[e] * (zv[mm][e] * sigmoidf_(zv[mm][e])));
            }
        }
    }
}

template <int PRO, int EPI, int KS, int NST>
__global__ __launch_bounds__(256, 2) void k_gemv_mfma(GemvMultiArgs a) {
    constexpr int U = kStage, NB = 4 / KS;   // NB row blocks per workgroup
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    typedef float f4 __attribute__((ext_vector_type(4)));
    extern __shared__ __align__(16) unsigned char smem[];
    float* red = (float*)smem;                        // 16 floats
    _Float16* xs = (_Float16*)(smem + 64);            // [M][K]
    const int K = a.K, G = K / 32, M = a.M, rows = a.rows;
    f4* part = (f4*)(smem + 64 + (size_t)2 * M * (K + kMfmaPad));   // [4 waves][64 lanes], KS > 1
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar branches
    const int c = lane & 15, q = lane >> 4;

    mfma_prologue<32 * KS * NST * U, PRO>(a, xs, red);
    __syncthreads();

    const int nrb = (rows + 15) / 16;
    // B operand: input min(c, M - 1) (columns past M are computed and dropped)
    const _Float16* xrow = xs + min(c, M - 1) * (K + kMfmaPad) + 8 * q;
    const NibK nk;
    const h2 off_lo = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 off_hi = {(_Float16)-72.0f, (_Float16)-72.0f};
    const f4 zero = {0.f, 0.f, 0.f, 0.f};
    struct Stage {
        u32x4 w[U / 4];     // row c, groups g0 + 4h + q (h < U/4), all four dwords
        uint4 s;            // row c: fp16 scales of groups g0 .. g0 + U - 1
    };
    const int gbeg = (wave % KS) * (NST * U);   // NST stages of U groups per wave
    // persistent: workgroup units (NB row blocks each) in turn, so that a
    // launch of one round of resident workgroups covers every row block
    const int nunits = (nrb + NB - 1) / NB;
    for (int unit = blockIdx.x; unit < nunits; unit += gridDim.x) {
        const int blk = unit * NB + wave / KS;
        const bool live = blk < nrb;                       // uniform over the KS waves of a block
        const int r0 = blk * 16;
        const int row = min(r0 + c, rows - 1);
        // codes: lane (c, q) loads row c's group g + q whole (16 bytes) and four
        // lane-row swaps hand each lane its dword of every group (see compute)
        const u32x4* arow = (const u32x4*)(a.codes + (int64_t)row * G * 4) + q;
        const uint16_t* srow = a.scales + (int64_t)row * G;
        auto load = [&](Stage& st, int sidx) {
            const int g0 = gbeg + sidx * U;
#pragma unroll
            for (int h = 0; h < U / 4; ++h) st.w[h] = arow[g0 + 4 * h];   // plain loads: see the head below
            st.s = *(const uint4*)(srow + g0);
        };
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        auto compute = [&](const Stage& st, int sidx) {
            const int g0 = gbeg + sidx * U;
            // the stage's input fragments first (LDS latency once per stage), then
            // the products back to back, then the scales
            uint4 xb[U];
#pragma unroll
            for (int j = 0; j < U; ++j) xb[j] = *(const uint4*)(xrow + 32 * (g0 + j));
            asm volatile("" ::: "memory");   // issued together, before the products
            // 4 x 4 transpose across the lane rows (16 lanes each): lane row t
            // holds dwords 0..3 of group g0 + 4h + t; after two 32-lane and two
            // 16-lane swaps, word j of lane row q is dword q of group g0 + 4h + j
            uint32_t wd[U];
#pragma unroll
            for (int h = 0; h < U / 4; ++h) {
                const auto ab = __builtin_amdgcn_permlane32_swap(st.w[h][0], st.w[h][2], false, false);
                const auto cd = __builtin_amdgcn_permlane32_swap(st.w[h][1], st.w[h][3], false, false);
                const auto t01 = __builtin_amdgcn_permlane16_swap(ab[0], cd[0], false, false);
                const auto t23 = __builtin_amdgcn_permlane16_swap(ab[1], cd[1], false, false);
                wd[4 * h] = t01[0];
                wd[4 * h + 1] = t01[1];
                wd[4 * h + 2] = t23[0];
                wd[4 * h + 3] = t23[1];
            }
            f4 d[U];
#pragma unroll
            for (int j = 0; j < U; ++j) {
                // exact codes: lo slots 1024 + n - 1032, hi slots (1024 + 16 n) / 16 - 72
                const uint32_t w = wd[j], w8 = w >> 8;
                const h2 p0 = as_h2((w & nk.lo) | nk.e) + off_lo;
                const h2 p1 = __builtin_elementwise_fma(as_h2((w & nk.hi) | nk.e), sixteenth, off_hi);
                const h2 p2 = as_h2((w8 & nk.lo) | nk.e) + off_lo;
                const h2 p3 = __builtin_elementwise_fma(as_h2((w8 & nk.hi) | nk.e), sixteenth, off_hi);
                const h8 av = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
                // D = X W^T: lane (c, q) gets inputs 4 q .. 4 q + 3 at row c
                d[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, xb[j]), av, zero, 0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < U; ++j) {
                const uint32_t sw = (j >> 1) == 0 ? st.s.x : (j >> 1) == 1 ? st.s.y : (j >> 1) == 2 ? st.s.z : st.s.w;
                const float sc = (float)as_h2(sw)[j & 1];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) acc[rr] += sc * d[j][rr];
            }
        };
        if (live) {
            // RING register sets used in turn, each refilled right after use, in
            // straight-line code (a loop header would merge the wait counts); loads
            // past the last stage re-read it so every step issues the same ones
            constexpr int RING = 5;
            Stage ring[RING];
#pragma unroll
            for (int k = 0; k < RING - 1; ++k) load(ring[k], k < NST ? k : NST - 1);
#pragma unroll
            for (int sidx = 0; sidx < NST; ++sidx) {
                load(ring[(sidx + RING - 1) % RING], sidx + RING - 1 < NST ? sidx + RING - 1 : NST - 1);
                asm volatile("" ::: "memory");   // keep each stage's loads in their place
                compute(ring[sidx % RING], sidx);
            }
        }
        // lane (c, q): inputs 4 q + rr at row r0 + c (M <= 4: the q = 0 lanes)
        bool out = live && q == 0;
        if (KS > 1) {
            part[wave * 64 + lane] = f4{acc[0], acc[1], acc[2], acc[3]};
            __syncthreads();
            if (wave % KS == 0) {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) acc[rr] = 0.f;
#pragma unroll
                for (int t = 0; t < KS; ++t) {
                    const f4 v = part[(wave + t) * 64 + lane];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) acc[rr] += v[rr];
                }
            } else {
                out = false;
            }
            __syncthreads();   // part[] is reused by the next unit
        }
        if (EPI == EPI_SWIGLU) {
            // interleaved gate/up rows: even lane c holds gate row r0 + c, the
            // next lane its up row
            float up[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) up[rr] = __shfl_down(acc[rr], 1, 64);
            if (out && (c & 1) == 0 && r0 + c + 1 < rows) {
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    if (m < M) {
                        const float gg = acc[m];
                        a.hout[m * a.so + ((r0 + c) >> 1)] = (_Float16)(gg * sigmoidf_(gg) * up[m]);
                    }
            }
        } else if (out && r0 + c < rows) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
                if (m < M) {
                    if (EPI == EPI_STORE) a.y[m * a.sy + r0 + c] = acc[m];
                    else a.y[m * a.sy + r0 + c] += acc[m];
                }
        }
    }
}

// int8 head over M <= 4 vectors on the matrix cores (row length H, a compile-
// time multiple of 256).  A wave takes blocks of 16 rows; per 64-byte span of
// a row (64 codes), lane (c, q) loads bytes 16 q .. 16 q + 15 of row c, and a
// 4 x 4 transpose across the lane rows (two 32-lane and two 16-lane swaps)
// leaves word j of lane row q = codes 16 j + 4 q .. + 3 of row c: the B
// operand of v_mfma_f32_16x16x16_f16 j (exact codes as fp16); the A operand
// is input c at the same four positions, from LDS.  The product D = X W^T
// gives lane (c, q) the logits of inputs 4 q .. 4 q + 3 at row c, so a lane
// needs only its own row's fp16 group scales.  Stages of SPS spans (2 SPS
// groups) run RING - 1 ahead in a ring of RING register sets, unrolled by RING
// so that no copy moves a set.  Each load instruction takes 64 bytes of each
// of 16 rows; plain loads serve that pattern faster than non-temporal ones
// (head 394 -> 297 us, M = 4 FFN gate/up 32.3 -> 27.9 us, with the same HBM
// bytes fetched), in this kernel and in k_gemv_mfma.  At the 27B width a
// stage takes 512 bytes of each row, one stage ahead (SPS 8, RING 2): longer
// runs per row than 128 bytes four stages ahead (SPS 2, RING 5), 299 -> 257
// us for the same bytes in flight (SPS 4: 272 us, SPS 16 or 20: 272, 300 us;
// three waves per SIMD at SPS 8: 259 us).
// Results: logits [M][V] and per-workgroup best value and index per vector
// (lowest index on ties), a.nparts partial slots per vector as k_head_multi
// (slots past the grid hold -inf).
template <int H, int SPS, int RING>
__global__ __launch_bounds__(256, 2) void k_head_mfma(HeadMultiArgs a) {
    constexpr int MAXM = 4, GR = H / 32, NSP = H / 64, NST = NSP / SPS;   // spans per stage, stages per row block
    static_assert(NSP % SPS == 0, "row length");
    typedef float f4 __attribute__((ext_vector_type(4)));
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    extern __shared__ __align__(16) unsigned char smem[];
    float* red = (float*)smem;
    _Float16* xs = (_Float16*)(smem + 64);   // [M][H + kMfmaPad]
    __shared__ float bv_s[MAXM][4];
    __shared__ int bi_s[MAXM][4];
    {
        GemvMultiArgs g{};
        g.K = H;
        g.M = a.M;
        g.x = a.x;
        g.sx = H;
        g.nw = a.nw;
        g.eps = a.eps;
        mfma_prologue<H, PRO_NORM>(g, xs, red);
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane & 15, q = lane >> 4;
    const int M = a.M, V = a.V;
    const int nrb = (V + 15) / 16;
    const _Float16* xrow = xs + min(c, M - 1) * (H + kMfmaPad) + 4 * q;
    const h2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
    float best[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    int besti[4] = {0x7fffffff, 0x7fffffff, 0x7fffffff, 0x7fffffff};
    struct Stage {
        u32x4 w[SPS];       // row c: span bytes 16 q .. 16 q + 15 of each span
        uint32_t s[SPS];    // row c: fp16 scales of the stage's 2 SPS groups
    };
    for (int rb = blockIdx.x * 4 + wave; rb < nrb; rb += gridDim.x * 4) {
        const int r0 = rb * 16;
        const int row = min(r0 + c, V - 1);
        const u32x4* arow = (const u32x4*)(a.codes + (int64_t)row * H) + q;
        const uint16_t* srow = a.scales + (int64_t)row * GR;
        auto load = [&](Stage& st, int sidx) {
#pragma unroll
            for (int h = 0; h < SPS; ++h) st.w[h] = arow[4 * (sidx * SPS + h)];
            const uint32_t* sp = (const uint32_t*)(srow + 2 * SPS * sidx);
#pragma unroll
            for (int h = 0; h < SPS; ++h) st.s[h] = sp[h];
        };
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        const f4 zero = {0.f, 0.f, 0.f, 0.f};
        auto compute = [&](const Stage& st, int sidx) {
#pragma unroll
            for (int h = 0; h < SPS; ++h) {
                const int k0 = 64 * (sidx * SPS + h);
                uint2 xb[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) xb[j] = *(const uint2*)(xrow + k0 + 16 * j);
                const auto ab = __builtin_amdgcn_permlane32_swap(st.w[h][0], st.w[h][2], false, false);
                const auto cd = __builtin_amdgcn_permlane32_swap(st.w[h][1], st.w[h][3], false, false);
                const auto t01 = __builtin_amdgcn_permlane16_swap(ab[0], cd[0], false, false);
                const auto t23 = __builtin_amdgcn_permlane16_swap(ab[1], cd[1], false, false);
                const uint32_t wd[4] = {t01[0], t01[1], t23[0], t23[1]};
                f4 d[2];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t b = wd[j] ^ 0x80808080u;
                    const h2 p01 = as_h2(__builtin_amdgcn_perm(0x64646464u, b, 0x04010400u)) - off;
                    const h2 p23 = as_h2(__builtin_amdgcn_perm(0x64646464u, b, 0x04030402u)) - off;
                    const h4 wv = {p01[0], p01[1], p23[0], p23[1]};
                    d[j >> 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4, xb[j]), wv,
                                                                     (j & 1) ? d[j >> 1] : zero, 0, 0, 0);
                }
                // groups 2 h and 2 h + 1 of the stage: this row's scales
                const h2 sc = as_h2(st.s[h]);
#pragma unroll
                for (int gg = 0; gg < 2; ++gg)
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) acc[rr] += (float)sc[gg] * d[gg][rr];
            }
        };
        // loads past the last stage re-read it, so every step issues the same ones
        Stage ring[RING];
#pragma unroll
        for (int k = 0; k < RING - 1; ++k) load(ring[k], min(k, NST - 1));
        for (int sidx = 0;; sidx += RING) {
#pragma unroll
            for (int k = 0; k < RING; ++k) {
                load(ring[(k + RING - 1) % RING], min(sidx + k + RING - 1, NST - 1));
                asm volatile("" ::: "memory");
                compute(ring[k], sidx + k);
                if (sidx + k + 1 >= NST) break;
            }
            if (sidx + RING >= NST) break;
        }
        // lane (c, q): inputs 4 q + rr at row r0 + c
        const int rowv = r0 + c;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int m = 4 * q + rr;
            if (m < M && rowv < V) {
                if (a.logits) a.logits[(int64_t)m * V + rowv] = acc[rr];
                if (better(acc[rr], rowv, best[rr], besti[rr])) { best[rr] = acc[rr]; besti[rr] = rowv; }
            }
        }
    }
    // per input (lanes q = 0, slot rr): best over the 16 rows of the lane row, then the waves
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int o = 1; o <= 8; o <<= 1) {
            const float ov = __shfl_xor(best[rr], o, 64);
            const int oi = __shfl_xor(besti[rr], o, 64);
            if (better(ov, oi, best[rr], besti[rr])) { best[rr] = ov; besti[rr] = oi; }
        }
    if (lane == 0) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            bv_s[rr][wave] = best[rr];
            bi_s[rr][wave] = besti[rr];
        }
    }
    __syncthreads();
    if (threadIdx.x < M) {
        const int m = threadIdx.x;
        float b = bv_s[m][0];
        int bi = bi_s[m][0];
        for (int w = 1; w < 4; ++w)
            if (better(bv_s[m][w], bi_s[m][w], b, bi)) { b = bv_s[m][w]; bi = bi_s[m][w]; }
        a.part_val[m * a.nparts + blockIdx.x] = b;
        a.part_idx[m * a.nparts + blockIdx.x] = bi;
        // slots past the grid: empty (never better than a real partial)
        for (int p = blockIdx.x + gridDim.x; p < a.nparts; p += gridDim.x) {
            a.part_val[m * a.nparts + p] = -INFINITY;
            a.part_idx[m * a.nparts + p] = 0x7fffffff;
        }
    }
}

// int8 head over M vectors (per-vector logits and per-block argmax partials)
__global__ __launch_bounds__(256) void k_head_multi(HeadMultiArgs a) {
    constexpr int MAXM = 4;
    extern __shared__ __align__(16) unsigned char smem[];
    float* red = (float*)smem;
    _Float16* xs = (_Float16*)(smem + 64);   // [M][H]
    __shared__ float bv_s[MAXM][4];
    __shared__ int bi_s[MAXM][4];
    {
        GemvMultiArgs g{};
        g.K = a.H;
        g.M = a.M;
        g.x = a.x;
        g.sx = a.H;
        g.nw = a.nw;
        g.eps = a.eps;
        multi_prologue<MAXM>(PRO_NORM, g, xs, red);
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H = a.H, M = a.M;
    const int nchunk = H >> 4;
    const int g_row = H >> 5;
    float best[MAXM];
    int besti[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) { best[m] = -INFINITY; besti[m] = 0x7fffffff; }
    for (int r = blockIdx.x * 4 + wave; r < a.V; r += gridDim.x * 4) {
        const uint4* c0 = (const uint4*)(a.codes + (int64_t)r * H);
        const uint16_t* s0 = a.scales + (int64_t)r * g_row;
        float acc[MAXM];
#pragma unroll
        for (int m = 0; m < MAXM; ++m) acc[m] = 0.f;
        for (int c = lane; c < nchunk; c += 64) {
            const uint4 w = c0[c];
            const float sc = half_bits_to_float(s0[c >> 1]);
#pragma unroll
            for (int m = 0; m < MAXM; ++m) {
                if (m < M) {
                    const uint4* xv = (const uint4*)(xs + m * H);
                    const uint4 xa = xv[2 * c], xb = xv[2 * c + 1];
                    float p = 0.f;
                    i8_dot4(w.x, xa.x, xa.y, p);
                    i8_dot4(w.y, xa.z, xa.w, p);
                    i8_dot4(w.z, xb.x, xb.y, p);
                    i8_dot4(w.w, xb.z, xb.w, p);
                    acc[m] += sc * p;
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            if (m < M) {
                const float v = wave_sum_fast(acc[m]);
                if (lane == 0) a.logits[(int64_t)m * a.V + r] = v;
                if (better(v, r, best[m], besti[m])) { best[m] = v; besti[m] = r; }
            }
        }
    }
    if (lane == 0)
#pragma unroll
        for (int m = 0; m < MAXM; ++m) { bv_s[m][wave] = best[m]; bi_s[m][wave] = besti[m]; }
    __syncthreads();
    if (threadIdx.x < M) {
        const int m = threadIdx.x;
        float b = bv_s[m][0];
        int bi = bi_s[m][0];
        for (int w = 1; w < 4; ++w)
            if (better(bv_s[m][w], bi_s[m][w], b, bi)) { b = bv_s[m][w]; bi = bi_s[m][w]; }
        a.part_val[m * gridDim.x + blockIdx.x] = b;
        a.part_idx[m * gridDim.x + blockIdx.x] = bi;
    }
}

// final argmax over the per-block results; feeds the next embedding and the
// greedy output ring, and advances the position
__global__ __launch_bounds__(256) void k_head_final(const float* pv, const int32_t* pi, int n, Ctl* ctl,
                                                     int32_t* ring, int ring_cap) {
    __shared__ float sv[256];
    __shared__ int si[256];
    float b = -INFINITY;
    int bi = 0x7fffffff;
    for (int i = threadIdx.x; i < n; i += 256)
        if (better(pv[i], pi[i], b, bi)) { b = pv[i]; bi = pi[i]; }
    sv[threadIdx.x] = b;
    si[threadIdx.x] = bi;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (threadIdx.x < s && better(sv[threadIdx.x + s], si[threadIdx.x + s], sv[threadIdx.x], si[threadIdx.x])) {
            sv[threadIdx.x] = sv[threadIdx.x + s];
            si[threadIdx.x] = si[threadIdx.x + s];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        int tok = si[0] == 0x7fffffff ? 0 : si[0];
        ctl->argmax = tok;
        ctl->token = tok;
        if (ring && ctl->nstep < ring_cap) ring[ctl->nstep] = tok;
        ctl->nstep += 1;
        ctl->pos += 1;
    }
}

}  // namespace

int gemv_blocks(int rows) {
    const int npairs = (rows + 1) / 2;
    const int max_waves = 4096;
    const int ppw = (npairs + max_waves - 1) / max_waves;
    const int waves = (npairs + ppw - 1) / ppw;
    return (waves + 3) / 4;
}

int head_blocks(int V) { return gemv_blocks(V); }

// workgroups of 256 threads of fn with shm bytes of dynamic LDS that the
// current device holds at once (0 if the runtime cannot tell); cached per
// (kernel, LDS size)
int resident_blocks(const void* fn, size_t shm) {
    struct Entry { const void* fn; size_t shm; int dev, n; };
    static Entry cache[64];
    static int ncache = 0;
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < ncache; ++i)
        if (cache[i].fn == fn && cache[i].shm == shm && cache[i].dev == dev) return cache[i].n;
    int cus = 0, nb = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, 256, shm) != hipSuccess)
        return 0;
    const int n = nb * cus;
    if (ncache < 64) cache[ncache++] = Entry{fn, shm, dev, n};
    return n;
}

// the mapped head over its shorter id list: one round of two workgroups per
// CU (measured 57 us for 65,536 rows against 65 us at the 1024 workgroups of
// head_blocks)
int draft_head_blocks(int V) { return std::min(head_blocks(V), 512); }

namespace {

int gcd_int(int a, int b) { return b ? gcd_int(b, a % b) : a; }

// rows per block and groups per lane of the streaming kernel for row length K
void stream_shape(int K, int& R, int& NF) {
    const int G = K / 32;
    R = 64 / gcd_int(64, G);
    if (R < 2) R = 2;
    NF = R * G / 64;
}

// 4-wave workgroups of a streaming launch over nrb row blocks: max_waves waves
// (or one per block), unless that would take more than kStreamMaxPer blocks per
// wave.  The per-wave block counts may differ by one: evening them out with
// fewer waves left part of the chip idle (GDN in-proj: 221 of 256 CUs).
int stream_grid(int nrb, int max_waves) {
    if (nrb > max_waves * kStreamMaxPer) max_waves = (nrb + kStreamMaxPer - 1) / kStreamMaxPer;
    const int waves = nrb < max_waves ? nrb : max_waves;
    return (waves + 3) / 4;
}

int stream_blocks(int rows, int R, int NF) {
    const int nrb = rows / R;
    // LDS-input form: as many waves as the compiled occupancy holds on 256 CUs
    // (4 SIMDs each); register-resident form: about one workgroup per CU
    // while the ring covers the rows in at most kStreamMaxPer steps, two for
    // more rows; long rows (NF > 8): up to 4096 waves of one block each
    if (stream_lds_x(NF)) return stream_grid(nrb, 1024 * stream_simd_waves(NF));
    return stream_grid(nrb, NF > 8 ? 4096 : nrb <= 1024 * kStreamMaxPer ? 1024 : 2048);
}

// the multi-input kernel: two workgroups per CU for short rows
int multi_blocks(int rows, int R, int NF) { return stream_grid(rows / R, NF <= 8 ? 2048 : 4096); }

template <int R, int NF>
hipError_t launch_stream(int pro, int epi, const GemvArgs& a, hipStream_t s) {
    const size_t shm = 64 + (size_t)xs_len<true>(a.K) * 2;
    const dim3 grid(stream_blocks(a.rows, R, NF)), block(256);
#define AW4_STREAM_CASE(P, E)                                                         \
    if (pro == P && epi == E) {                                                       \
        hipLaunchKernelGGL((k_gemv_stream<R, NF, P, E>), grid, block, shm, s, a);     \
        return hipGetLastError();                                                     \
    }
    AW4_STREAM_CASE(PRO_NORM, EPI_STORE)
    AW4_STREAM_CASE(PRO_NORM, EPI_SWIGLU)
    AW4_STREAM_CASE(PRO_GATED, EPI_RESID)
    AW4_STREAM_CASE(PRO_LOADH, EPI_RESID)
    if constexpr (R == 2 && NF == 10) {   // draft-head fuse, K 10240
        AW4_STREAM_CASE(PRO_LOADH, EPI_STORE)
    }
#undef AW4_STREAM_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_generic(int pro, int epi, const GemvArgs& a, hipStream_t s) {
    const size_t shm = 64 + (size_t)a.K * 2;
    const dim3 grid(gemv_blocks(a.rows)), block(256);
#define AW4_GEMV_CASE(P, E)                                                     \
    if (pro == P && epi == E) {                                                 \
        hipLaunchKernelGGL((k_gemv_w4<P, E>), grid, block, shm, s, a);          \
        return hipGetLastError();                                               \
    }
    AW4_GEMV_CASE(PRO_NORM, EPI_STORE)
    AW4_GEMV_CASE(PRO_NORM, EPI_SWIGLU)
    AW4_GEMV_CASE(PRO_GATED, EPI_RESID)
    AW4_GEMV_CASE(PRO_LOADH, EPI_RESID)
    AW4_GEMV_CASE(PRO_LOADH, EPI_STORE)
#undef AW4_GEMV_CASE
    return hipErrorInvalidValue;
}

}  // namespace

// Streaming kernel for the row lengths it is instantiated for (the 27B shapes
// and the small test shapes) when the row count splits into whole row blocks;
// the generic kernel otherwise.
hipError_t launch_gemv(int pro, int epi, const GemvArgs& a, hipStream_t s) {
    int R, NF;
    stream_shape(a.K, R, NF);
    bool ok = a.rows % R == 0;
    if (pro == PRO_GATED) {
        // the compile-time gated prologue gives each head d / E lanes of one wave
        const int E = a.K >= 256 ? a.K / 256 : 1;
        ok = ok && E <= a.gated_d && a.gated_d / E <= 64 && (a.K < 256 || a.K % 256 == 0);
    }
    if (ok) {
#define AW4_SHAPE(RR, FF) \
        if (R == RR && NF == FF) return launch_stream<RR, FF>(pro, epi, a, s);
        AW4_SHAPE(2, 5)     // K = 5120
        AW4_SHAPE(2, 4)     // K = 4096
        AW4_SHAPE(2, 6)     // K = 6144
        AW4_SHAPE(2, 17)    // K = 17408
        AW4_SHAPE(2, 10)    // K = 10240 (draft-head fuse)
        AW4_SHAPE(4, 1)     // K = 512
        AW4_SHAPE(4, 3)     // K = 1536
        AW4_SHAPE(8, 1)     // K = 256
        AW4_SHAPE(16, 1)    // K = 128
#undef AW4_SHAPE
    }
    return launch_generic(pro, epi, a, s);
}

namespace {
template <int R, int NF>
hipError_t launch_multi_rnf(int pro, int epi, const GemvMultiArgs& a, hipStream_t s) {
    const size_t kp = NF <= 8 ? (size_t)(a.K / 32) * 40 : (size_t)a.K;   // the kernel's kPad
    const size_t shm = 64 + kp * 2 * (size_t)a.M;
    const dim3 grid(multi_blocks(a.rows + R - 1, R, NF)), block(256);
#define AW4_MULTI_CASE(P, E)                                                                        \
    if (pro == P && epi == E) {                                                                     \
        if (shm > 65536) {                                                                          \
            hipError_t e = hipFuncSetAttribute((const void*)k_gemv_multi<R, NF, P, E>,              \
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm); \
            if (e != hipSuccess) return e;                                                          \
        }                                                                                           \
        hipLaunchKernelGGL((k_gemv_multi<R, NF, P, E>), grid, block, shm, s, a);                    \
        return hipGetLastError();                                                                   \
    }
    AW4_MULTI_CASE(PRO_NORM, EPI_STORE)
    AW4_MULTI_CASE(PRO_NORM, EPI_SWIGLU)
    AW4_MULTI_CASE(PRO_GATED, EPI_RESID)
    AW4_MULTI_CASE(PRO_LOADH, EPI_RESID)
#undef AW4_MULTI_CASE
    return hipErrorInvalidValue;
}
}  // namespace

namespace {
template <int P, int E, int KS, int NST>
hipError_t launch_mfma(const GemvMultiArgs& a, hipStream_t s) {
    const int nrb = (a.rows + 15) / 16;
    const int nunits = (nrb + 4 / KS - 1) / (4 / KS);
    const size_t shm = 64 + (size_t)2 * a.M * (a.K + kMfmaPad) + (KS > 1 ? 4 * 64 * 16 : 0);
    const void* fn = (const void*)k_gemv_mfma<P, E, KS, NST>;
    if (shm > 65536) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        if (e != hipSuccess) return e;
    }
    // one round of resident workgroups, each taking units in turn: a partial
    // second round ran on a mostly idle chip
    const int res = resident_blocks(fn, shm);
    const dim3 grid(res > 0 && res < nunits ? res : nunits), block(256);
    hipLaunchKernelGGL((k_gemv_mfma<P, E, KS, NST>), grid, block, shm, s, a);
    return hipGetLastError();
}

// the instantiated (prologue, epilogue, waves per block, stages per wave):
// the 27B-shape matrices and the small test stack; true if launched
bool try_mfma(int pro, int epi, int ks, int nst, const GemvMultiArgs& a, hipStream_t s, hipError_t& err) {
#define AW4_MFMA(P, E, KS, NST)                              \
    if (pro == P && epi == E && ks == KS && nst == NST) {    \
        err = launch_mfma<P, E, KS, NST>(a, s);              \
        return true;                                         \
    }
    AW4_MFMA(PRO_NORM, EPI_SWIGLU, 4, 5)    // FFN gate/up, K 5120
    AW4_MFMA(PRO_NORM, EPI_STORE, 4, 5)     // mixer in-projections, K 5120
    AW4_MFMA(PRO_GATED, EPI_RESID, 4, 4)    // GDN out-projection, K 4096
    AW4_MFMA(PRO_LOADH, EPI_RESID, 4, 6)    // attention o-projection, K 6144
    AW4_MFMA(PRO_LOADH, EPI_RESID, 4, 17)   // FFN down, K 17408
    AW4_MFMA(PRO_LOADH, EPI_RESID, 2, 34)   // FFN down when one workgroup fills a CU's LDS
    AW4_MFMA(PRO_LOADH, EPI_STORE, 4, 10)   // draft-head fuse, K 10240
    AW4_MFMA(PRO_LOADH, EPI_STORE, 4, 1)    // the same on the small stack (K 1024)
    AW4_MFMA(PRO_NORM, EPI_SWIGLU, 2, 1)    // small stack (K 512, 1536, 256)
    AW4_MFMA(PRO_NORM, EPI_STORE, 2, 1)
    AW4_MFMA(PRO_LOADH, EPI_RESID, 2, 3)
    AW4_MFMA(PRO_GATED, EPI_RESID, 1, 1)
    AW4_MFMA(PRO_LOADH, EPI_RESID, 1, 1)
#undef AW4_MFMA
    return false;
}
}  // namespace

// M <= 4 vectors: on the matrix cores when the groups split into whole stages
// (every 27B-shape matrix), else the dot-product kernel.  Row blocks that
// would leave the chip short of waves split their groups over 2 or 4 waves.
hipError_t launch_gemv_multi(int pro, int epi, const GemvMultiArgs& a, hipStream_t s) {
    if (a.M < 1 || a.M > 4) return hipErrorInvalidValue;
    int R, NF;
    stream_shape(a.K, R, NF);
    if (pro == PRO_GATED && (a.gated_d <= 0 || a.K % a.gated_d)) return hipErrorInvalidValue;
    const int G = a.K / 32;
    if (a.K % 32 == 0 && G % kStage == 0 && a.rows >= 1) {
        const int nrb = (a.rows + 15) / 16;
        // at least two waves per row block: with one, the stage offsets are
        // compile-time constants and the compiler merges the ring's loads
        // until the registers spill.  Four where the groups allow it: the
        // resident workgroups take row blocks in turn, and the finer unit
        // evens out their counts (2176 gate/up row blocks in units of two
        // over 768 workgroups left a 41% tail)
        int ks = G % (4 * kStage) == 0 ? 4 : G % (2 * kStage) == 0 ? 2 : 1;
        // an input image above half the LDS leaves one workgroup per CU: then
        // two waves per row block keep the grid within one round of CUs
        if (ks == 4 && (size_t)2 * a.M * a.K > 80 * 1024) ks = 2;
        hipError_t err;
        if (try_mfma(pro, epi, ks, G / (ks * kStage), a, s, err)) return err;
    }
#define AW4_SHAPE(RR, FF) \
    if (R == RR && NF == FF) return launch_multi_rnf<RR, FF>(pro, epi, a, s);
    AW4_SHAPE(2, 5)
    AW4_SHAPE(2, 4)
    AW4_SHAPE(2, 6)
    AW4_SHAPE(2, 17)
    AW4_SHAPE(4, 1)
    AW4_SHAPE(4, 3)
    AW4_SHAPE(8, 1)
    AW4_SHAPE(16, 1)
    AW4_SHAPE(32, 3)
#undef AW4_SHAPE
    return hipErrorInvalidValue;
}

hipError_t launch_head_multi(const HeadMultiArgs& a, hipStream_t s) {
    if (a.M < 1 || a.M > 4) return hipErrorInvalidValue;
    if (a.H == 5120 || a.H == 512) {
        // the matrix-core form (27B and toy widths); one partial per workgroup
        // and vector as below, head_blocks(V) workgroups
        const size_t shm = 64 + (size_t)2 * a.M * (a.H + kMfmaPad);
        const void* fn = a.H == 5120 ? (const void*)k_head_mfma<5120, 8, 2> : (const void*)k_head_mfma<512, 2, 5>;
        if (shm > 65536) {
            hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
            if (e != hipSuccess) return e;
        }
        // one round of resident workgroups (a partial second round ran on a
        // mostly idle chip); partial slots past the grid are filled empty
        HeadMultiArgs b = a;
        b.nparts = head_blocks(a.V);
        const int res = resident_blocks(fn, shm);
        const dim3 grid(res > 0 && res < b.nparts ? res : b.nparts);
        if (a.H == 5120) hipLaunchKernelGGL((k_head_mfma<5120, 8, 2>), grid, dim3(256), shm, s, b);
        else hipLaunchKernelGGL((k_head_mfma<512, 2, 5>), grid, dim3(256), shm, s, b);
        return hipGetLastError();
    }
    const size_t shm = 64 + (size_t)a.H * 2 * (size_t)a.M;
    if (shm > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)k_head_multi, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_head_multi, dim3(head_blocks(a.V)), dim3(256), shm, s, a);
    return hipGetLastError();
}

hipError_t launch_head(const HeadArgs& a, hipStream_t s) {
    const size_t shm = 64 + (size_t)a.H * 2;
    if (a.H == 5120 && a.map) {
        hipLaunchKernelGGL((k_head_stream<5120, true>), dim3(draft_head_blocks(a.V)), dim3(256), shm, s, a);
    } else if (a.H == 5120) {
        hipLaunchKernelGGL((k_head_stream<5120, false>), dim3(head_blocks(a.V)), dim3(256), shm, s, a);
    }
    else
        hipLaunchKernelGGL(k_head_i8, dim3(a.map ? draft_head_blocks(a.V) : head_blocks(a.V)), dim3(256), shm, s, a);
    return hipGetLastError();
}

hipError_t launch_head_final(const float* pv, const int32_t* pi, int n, Ctl* ctl, int32_t* ring, int ring_cap,
                             hipStream_t s) {
    hipLaunchKernelGGL(k_head_final, dim3(1), dim3(256), 0, s, pv, pi, n, ctl, ring, ring_cap);
    return hipGetLastError();
}

}  // namespace aw4

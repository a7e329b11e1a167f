// Small kernels: embedding, control-block updates, fills, and the group codec
// that packs fp32 weights into the GPU layouts.
//
// Codec (4-bit weights per page 1, dcwnkz.com "27B x 4 bit" estimate, and page
// 4, jdon.com W4A16; the int8 head follows the same recipe with qmax 127):
// per 32 consecutive inputs of a row, s = fp16(amax / qmax) with the quotient
// in fp32 and round-to-nearest-even, codes clamp(rint(w / s), -qmax, qmax),
// all codes 0 when s rounds to 0.
#include "aw4_internal.h"
#include "../../include/aw4.h"

namespace aw4 {
namespace {

__global__ void k_embed(const int8_t* __restrict__ codes, const uint16_t* __restrict__ scales, int H,
                        const Ctl* ctl, float* __restrict__ x) {
    const int64_t tok = ctl->token;
    for (int k = blockIdx.x * blockDim.x + threadIdx.x; k < H; k += gridDim.x * blockDim.x) {
        const float s = (float)__builtin_bit_cast(_Float16, scales[tok * (H / 32) + k / 32]);
        x[k] = (float)codes[tok * H + k] * s;
    }
}

__global__ void k_set_token(Ctl* ctl, int32_t token) { ctl->token = token; }

__global__ void k_embed_multi(const int8_t* __restrict__ codes, const uint16_t* __restrict__ scales, int H,
                              const Ctl* ctl, int M, float* __restrict__ x) {
    for (int m = 0; m < M; ++m) {
        const int64_t tok = ctl->vtok[m];
        for (int k = blockIdx.x * blockDim.x + threadIdx.x; k < H; k += gridDim.x * blockDim.x) {
            const float s = (float)__builtin_bit_cast(_Float16, scales[tok * (H / 32) + k / 32]);
            x[(int64_t)m * H + k] = (float)codes[tok * H + k] * s;
        }
    }
}

// token rows of a device id array, one workgroup per token
__global__ void k_embed_tokens(const int8_t* __restrict__ codes, const uint16_t* __restrict__ scales, int H,
                               const int32_t* tok, float* __restrict__ x) {
    const int m = blockIdx.x;
    const int64_t id = tok[m];
    for (int k = threadIdx.x; k < H; k += blockDim.x)
        x[(int64_t)m * H + k] = (float)codes[id * H + k] * (float)__builtin_bit_cast(_Float16, scales[id * (H / 32) + k / 32]);
}

struct BatchIn {
    int32_t tok[4];
    int32_t pos[4];
};

__global__ void k_set_batch(Ctl* ctl, BatchIn in) {
    for (int i = 0; i < 4; ++i) {
        ctl->btok[i] = in.tok[i];
        ctl->bpos[i] = in.pos[i];
    }
}

struct VerifyIn {
    int32_t tok[4];
    float u[4];
};

__global__ void k_set_verify(Ctl* ctl, VerifyIn in) {
    for (int i = 0; i < 4; ++i) {
        ctl->vtok[i] = in.tok[i];
        ctl->vu[i] = in.u[i];
        ctl->vout[i] = 0;
    }
    ctl->vn_acc = ctl->vn_out = ctl->vcommit = ctl->vresid_p = 0;
}

__global__ void k_advance(Ctl* ctl) { ctl->pos += 1; }

__global__ void k_set_ctl(Ctl* ctl, int32_t pos, int32_t token, int32_t nstep) {
    if (pos >= 0) ctl->pos = pos;
    if (token >= 0) ctl->token = token;
    if (nstep >= 0) ctl->nstep = nstep;
}

__global__ void k_fill_zero(uint32_t* p, uint64_t n) {
    for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

__global__ void k_copy_f32(float* dst, const float* src, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

// Plain streaming read for bandwidth reports: workgroup b reads the b-th
// contiguous chunk of per 16-byte words, eight 4 KB workgroup loads in flight
// (16-byte non-temporal loads, every wave load 1 KB contiguous), folds them
// into one word and writes it per workgroup so nothing is dropped.  Of the
// forms measured on the device (grid-wide stride with 2048 workgroups; chunks
// with 512 to 4096 workgroups; plain or non-temporal loads) this one, at 512
// workgroups, reads fastest.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void k_stream_read(const u32x4_t* __restrict__ src, uint64_t n16, uint64_t per,
                                                     uint32_t* sink) {
    constexpr int U = 8;
    uint32_t acc = 0;
    const uint64_t beg = blockIdx.x * per;
    const uint64_t end = beg + per < n16 ? beg + per : n16;
    uint64_t i = beg + threadIdx.x;
    for (; i + (U - 1) * 256 < end; i += U * 256) {
        u32x4_t v[U];
#pragma unroll
        for (int j = 0; j < U; ++j) v[j] = __builtin_nontemporal_load(src + i + j * 256);
#pragma unroll
        for (int j = 0; j < U; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
    }
    for (; i < end; i += 256) {
        const u32x4_t a = __builtin_nontemporal_load(src + i);
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
    for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
    if ((threadIdx.x & 63) == 0) atomicXor(&sink[blockIdx.x], acc);
}

__device__ __forceinline__ void quant_group32(const float* w, int qmax, int* c, uint16_t* sbits) {
    float amax = 0.f;
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(w[i]));
    const _Float16 sh = (_Float16)(amax / (float)qmax);
    const float s = (float)sh;
    for (int i = 0; i < 32; ++i) {
        float q = s == 0.f ? 0.f : rintf(w[i] / s);
        q = fminf(fmaxf(q, -(float)qmax), (float)qmax);
        c[i] = (int)q;
    }
    *sbits = __builtin_bit_cast(uint16_t, sh);
}

// one thread per (row, group of 32); dst rows are row_stride apart
__global__ void k_quant_w4(const float* __restrict__ src, int64_t nrows, int64_t cols, uint32_t* __restrict__ codes,
                           uint16_t* __restrict__ scales, int64_t row_stride) {
    const int64_t G = cols / 32;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < nrows * G;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = t / G, g = t % G;
        int c[32];
        uint16_t sb;
        quant_group32(src + r * cols + g * 32, 7, c, &sb);
        uint32_t* dst = codes + r * row_stride * (cols / 8) + g * 4;
        for (int m = 0; m < 4; ++m) {
            uint32_t w = 0;
            for (int e = 0; e < 8; ++e) w |= (uint32_t)((c[8 * m + e] + 8) & 15) << (4 * w4_slot(e));
            dst[m] = w;
        }
        scales[r * row_stride * G + g] = sb;
    }
}

__global__ void k_quant_i8(const float* __restrict__ src, int64_t nrows, int64_t cols, int8_t* __restrict__ codes,
                           uint16_t* __restrict__ scales) {
    const int64_t G = cols / 32;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < nrows * G;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = t / G, g = t % G;
        int c[32];
        uint16_t sb;
        quant_group32(src + r * cols + g * 32, 127, c, &sb);
        for (int i = 0; i < 32; ++i) codes[r * cols + g * 32 + i] = (int8_t)c[i];
        scales[r * G + g] = sb;
    }
}

int grid_for(int64_t n, int per_block = 256) {
    int64_t g = (n + per_block - 1) / per_block;
    if (g > 8192) g = 8192;
    if (g < 1) g = 1;
    return (int)g;
}

}  // namespace

hipError_t launch_embed(const int8_t* codes, const uint16_t* scales, int H, const Ctl* ctl, float* x,
                        hipStream_t s) {
    hipLaunchKernelGGL(k_embed, dim3(grid_for(H)), dim3(256), 0, s, codes, scales, H, ctl, x);
    return hipGetLastError();
}

hipError_t launch_embed_multi(const int8_t* codes, const uint16_t* scales, int H, const Ctl* ctl, int M, float* x,
                              hipStream_t s) {
    hipLaunchKernelGGL(k_embed_multi, dim3(grid_for(H)), dim3(256), 0, s, codes, scales, H, ctl, M, x);
    return hipGetLastError();
}

hipError_t launch_embed_tokens(const int8_t* codes, const uint16_t* scales, int H, const int32_t* tok, int M, float* x,
                               hipStream_t s) {
    hipLaunchKernelGGL(k_embed_tokens, dim3(M), dim3(256), 0, s, codes, scales, H, tok, x);
    return hipGetLastError();
}

hipError_t launch_set_batch(Ctl* ctl, const int32_t* tok, const int32_t* pos, hipStream_t s) {
    BatchIn in;
    for (int i = 0; i < 4; ++i) {
        in.tok[i] = tok[i];
        in.pos[i] = pos[i];
    }
    hipLaunchKernelGGL(k_set_batch, dim3(1), dim3(1), 0, s, ctl, in);
    return hipGetLastError();
}

hipError_t launch_set_verify(Ctl* ctl, const int32_t* tok, const float* u, hipStream_t s) {
    VerifyIn in;
    for (int i = 0; i < 4; ++i) {
        in.tok[i] = tok[i];
        in.u[i] = u[i];
    }
    hipLaunchKernelGGL(k_set_verify, dim3(1), dim3(1), 0, s, ctl, in);
    return hipGetLastError();
}

hipError_t launch_set_token(Ctl* ctl, int32_t token, hipStream_t s) {
    hipLaunchKernelGGL(k_set_token, dim3(1), dim3(1), 0, s, ctl, token);
    return hipGetLastError();
}

hipError_t launch_advance(Ctl* ctl, hipStream_t s) {
    hipLaunchKernelGGL(k_advance, dim3(1), dim3(1), 0, s, ctl);
    return hipGetLastError();
}

hipError_t launch_set_ctl(Ctl* ctl, int32_t pos, int32_t token, int32_t nstep, hipStream_t s) {
    hipLaunchKernelGGL(k_set_ctl, dim3(1), dim3(1), 0, s, ctl, pos, token, nstep);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, uint64_t bytes, hipStream_t s) {
    if (bytes % 4) return hipErrorInvalidValue;
    const uint64_t n = bytes / 4;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_zero, dim3(grid_for((int64_t)n)), dim3(256), 0, s, (uint32_t*)p, n);
    return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, uint64_t bytes, uint32_t* sink, int nblocks, hipStream_t s) {
    if (bytes % 16 || nblocks < 1) return hipErrorInvalidValue;
    const uint64_t n16 = bytes / 16;
    // chunks of whole 256-word workgroup loads that cover the range
    const uint64_t per = ((n16 + nblocks - 1) / nblocks + 255) / 256 * 256;
    hipLaunchKernelGGL(k_stream_read, dim3(nblocks), dim3(256), 0, s, (const u32x4_t*)src, n16, per, sink);
    return hipGetLastError();
}

hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t s) {
    hipLaunchKernelGGL(k_copy_f32, dim3(grid_for(n)), dim3(256), 0, s, dst, src, n);
    return hipGetLastError();
}

hipError_t launch_quant_w4(const float* src, int64_t nrows, int64_t cols, uint32_t* codes, uint16_t* scales,
                           int64_t row_stride, hipStream_t s) {
    hipLaunchKernelGGL(k_quant_w4, dim3(grid_for(nrows * (cols / 32))), dim3(256), 0, s, src, nrows, cols, codes,
                       scales, row_stride);
    return hipGetLastError();
}

hipError_t launch_quant_i8(const float* src, int64_t nrows, int64_t cols, int8_t* codes, uint16_t* scales,
                           hipStream_t s) {
    hipLaunchKernelGGL(k_quant_i8, dim3(grid_for(nrows * (cols / 32))), dim3(256), 0, s, src, nrows, cols, codes,
                       scales);
    return hipGetLastError();
}

}  // namespace aw4

// Streaming-read bandwidth of the device (the reference point beside the 8 TB/s
// peak in bandwidth reports): reps launches of k_stream_read over bytes at
// dev_src between two events on hip_stream, after one untimed launch; the
// average launch duration in microseconds.  dev_sink: at least 8 KB of device
// memory (one word per workgroup, 512 workgroups: 2 per compute unit).
extern "C" int aw4_time_stream_read(const void* dev_src, uint64_t bytes, void* dev_sink, void* hip_stream, int32_t reps,
                                    float* avg_us) {
    if (!dev_src || !dev_sink || !avg_us || reps < 1 || bytes < 16 || bytes % 16) return AW4_E_INVAL;
    hipStream_t s = (hipStream_t)hip_stream;
    constexpr int kBlocks = 512;
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return AW4_E_HIP;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return AW4_E_HIP;
    }
    bool ok = aw4::launch_stream_read(dev_src, bytes, (uint32_t*)dev_sink, kBlocks, s) == hipSuccess;
    ok = ok && hipEventRecord(e0, s) == hipSuccess;
    for (int i = 0; ok && i < reps; ++i) ok = aw4::launch_stream_read(dev_src, bytes, (uint32_t*)dev_sink, kBlocks, s) == hipSuccess;
    ok = ok && hipEventRecord(e1, s) == hipSuccess && hipEventSynchronize(e1) == hipSuccess;
    float ms = 0.f;
    ok = ok && hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (!ok) return AW4_E_HIP;
    *avg_us = ms * 1000.f / (float)reps;
    return AW4_OK;
}

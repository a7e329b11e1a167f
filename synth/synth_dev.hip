// Seeded synthetic-input generator, device (gfx950) implementation.
//
// Same definitions as synth_host.c (Philox4x32-10 of Salmon et al., SC'11;
// Irwin-Hall normals from twelve 16-bit uniforms), so that a tensor filled here
// equals, bit for bit, the tensor the host fills for the CPU oracle.  It holds
// none of the decode step's arithmetic and is not part of the product library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;

__device__ __forceinline__ void philox(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) { k0 += kW0; k1 += kW1; }
        uint32_t hi0 = __umulhi(kM0, c[0]), lo0 = kM0 * c[0];
        uint32_t hi1 = __umulhi(kM1, c[2]), lo1 = kM1 * c[2];
        uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
    }
}

__device__ __forceinline__ int32_t ih12(uint64_t seed, uint32_t stream, uint64_t i) {
    uint32_t a[4] = {(uint32_t)i, (uint32_t)(i >> 32), stream, 0u};
    uint32_t b[4] = {(uint32_t)i, (uint32_t)(i >> 32), stream, 1u};
    philox(a, (uint32_t)seed, (uint32_t)(seed >> 32));
    philox(b, (uint32_t)seed, (uint32_t)(seed >> 32));
    uint32_t w[6] = {a[0], a[1], a[2], a[3], b[0], b[1]};
    int32_t s = 0;
#pragma unroll
    for (int j = 0; j < 6; ++j) s += (int32_t)(w[j] & 0xFFFFu) + (int32_t)(w[j] >> 16);
    return s - 393210;
}

__device__ __forceinline__ uint32_t u32_at(uint64_t seed, uint32_t stream, uint64_t i) {
    uint32_t a[4] = {(uint32_t)i, (uint32_t)(i >> 32), stream, 2u};
    philox(a, (uint32_t)seed, (uint32_t)(seed >> 32));
    return a[0];
}

__global__ void k_normal(float* __restrict__ out, int64_t base, int64_t n, float sigma,
                         uint64_t seed, uint32_t stream) {
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n;
         e += (int64_t)gridDim.x * blockDim.x) {
        float z = __fmul_rn((float)ih12(seed, stream, (uint64_t)(base + e)), 1.0f / 65536.0f);
        out[e] = __fmul_rn(sigma, z);
    }
}

__global__ void k_codes(int8_t* __restrict__ out, int64_t i0, int64_t n, int32_t spread256,
                        int32_t qmax, uint64_t seed, uint32_t stream) {
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n;
         e += (int64_t)gridDim.x * blockDim.x) {
        int64_t v = (int64_t)ih12(seed, stream, (uint64_t)(i0 + e)) * spread256 + (1ll << 23);
        int64_t c = v >> 24;
        c = c > qmax ? qmax : c;
        c = c < -qmax ? -qmax : c;
        out[e] = (int8_t)c;
    }
}

__global__ void k_scale_bits(uint16_t* __restrict__ out, int64_t i0, int64_t n, uint32_t base_bits,
                             uint64_t seed, uint32_t stream) {
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n;
         e += (int64_t)gridDim.x * blockDim.x)
        out[e] = (uint16_t)(base_bits + (u32_at(seed, stream, (uint64_t)(i0 + e)) >> 28) - 8u);
}

__global__ void k_u32(uint32_t* __restrict__ out, int64_t i0, int64_t n, uint64_t seed,
                      uint32_t stream) {
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n;
         e += (int64_t)gridDim.x * blockDim.x)
        out[e] = u32_at(seed, stream, (uint64_t)(i0 + e));
}

__global__ void k_tokens(int32_t* __restrict__ out, int64_t i0, int64_t n, int32_t vocab,
                         uint64_t seed, uint32_t stream) {
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n;
         e += (int64_t)gridDim.x * blockDim.x)
        out[e] = (int32_t)(((uint64_t)u32_at(seed, stream, (uint64_t)(i0 + e)) * (uint64_t)vocab) >> 32);
}

int grid_for(int64_t n) {
    int64_t g = (n + 255) / 256;
    if (g > 65536) g = 65536;
    if (g < 1) g = 1;
    return (int)g;
}

}  // namespace

extern "C" {

// All pointers are device pointers; stream is a hipStream_t (null = default).
// Returns 0 on success or the hipError_t of the launch.
int aw4s_dev_normal_f32(float* out, int64_t row0, int64_t nrows, int64_t cols, float sigma,
                        uint64_t seed, uint32_t stream, void* hip_stream) {
    int64_t n = nrows * cols;
    if (n <= 0) return 0;
    k_normal<<<grid_for(n), 256, 0, (hipStream_t)hip_stream>>>(out, row0 * cols, n, sigma, seed, stream);
    return (int)hipGetLastError();
}

int aw4s_dev_codes_i8(int8_t* out, int64_t i0, int64_t n, int32_t spread256, int32_t qmax,
                      uint64_t seed, uint32_t stream, void* hip_stream) {
    if (n <= 0) return 0;
    k_codes<<<grid_for(n), 256, 0, (hipStream_t)hip_stream>>>(out, i0, n, spread256, qmax, seed, stream);
    return (int)hipGetLastError();
}

int aw4s_dev_scale_bits(uint16_t* out, int64_t i0, int64_t n, uint16_t base_bits, uint64_t seed,
                        uint32_t stream, void* hip_stream) {
    if (n <= 0) return 0;
    k_scale_bits<<<grid_for(n), 256, 0, (hipStream_t)hip_stream>>>(out, i0, n, base_bits, seed, stream);
    return (int)hipGetLastError();
}

int aw4s_dev_u32(uint32_t* out, int64_t i0, int64_t n, uint64_t seed, uint32_t stream, void* hip_stream) {
    if (n <= 0) return 0;
    k_u32<<<grid_for(n), 256, 0, (hipStream_t)hip_stream>>>(out, i0, n, seed, stream);
    return (int)hipGetLastError();
}

int aw4s_dev_tokens(int32_t* out, int64_t i0, int64_t n, int32_t vocab, uint64_t seed, uint32_t stream,
                    void* hip_stream) {
    if (n <= 0) return 0;
    k_tokens<<<grid_for(n), 256, 0, (hipStream_t)hip_stream>>>(out, i0, n, vocab, seed, stream);
    return (int)hipGetLastError();
}

}  // extern "C"

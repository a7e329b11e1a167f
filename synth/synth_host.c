/*
 * Seeded synthetic-input generator, host (CPU) implementation.
 *
 * This module produces the inputs that both the CPU oracle and the GPU path
 * consume: random weights, prompt tokens, uniforms, sign vectors and
 * synthetic cache contents.  It holds none of the decode step's arithmetic.
 *
 * Randomness: Philox4x32-10, the counter-based generator published by
 * Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as
 * 1, 2, 3" (SC'11).  A device implementation of the same definition lives in
 * synth_dev.hip; the two agree bit for bit because every value below is made
 * with integer arithmetic plus at most one IEEE fp32 multiply.
 *
 * Normal draws use the Irwin-Hall construction: the sum of twelve 16-bit
 * uniform integers, centred and divided by 2^16, has mean 0 and variance
 * 1 - 2^-32, and is exact in fp32.  sigma * z is the only rounding step.
 *
 * Counter layout for element index i of stream s under seed (k0, k1):
 *   normal  : blocks ctr = {i_lo, i_hi, s, 0} and {i_lo, i_hi, s, 1}; the
 *             first six 32-bit words give twelve 16-bit uniforms.
 *   uniform : block ctr = {i_lo, i_hi, s, 2}, word 0.
 */
#include <stdint.h>
#include <stddef.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void aw4s_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        if (r) { k0 += PHILOX_W0; k1 += PHILOX_W1; }
        uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static inline void block(uint64_t seed, uint32_t stream, uint64_t i, uint32_t purpose, uint32_t out[4]) {
    uint32_t ctr[4] = {(uint32_t)i, (uint32_t)(i >> 32), stream, purpose};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    aw4s_philox4x32_10(ctr, key, out);
}

/* Irwin-Hall integer: the sum of twelve 16-bit uniforms minus its mean
 * 12 * 32767.5 = 393210, an integer in [-393210, 393210]. */
static inline int32_t ih12(uint64_t seed, uint32_t stream, uint64_t i) {
    uint32_t a[4], b[4];
    block(seed, stream, i, 0u, a);
    block(seed, stream, i, 1u, b);
    uint32_t w[6] = {a[0], a[1], a[2], a[3], b[0], b[1]};
    int32_t s = 0;
    for (int j = 0; j < 6; ++j) s += (int32_t)(w[j] & 0xFFFFu) + (int32_t)(w[j] >> 16);
    return s - 393210;
}

uint32_t aw4s_u32_at(uint64_t seed, uint32_t stream, uint64_t i) {
    uint32_t a[4];
    block(seed, stream, i, 2u, a);
    return a[0];
}

int32_t aw4s_ih12_at(uint64_t seed, uint32_t stream, uint64_t i) { return ih12(seed, stream, i); }

/* out[r*cols + c] = sigma * z(seed, stream, (row0 + r) * cols + c) */
void aw4s_normal_f32(float* out, int64_t row0, int64_t nrows, int64_t cols, float sigma,
                     uint64_t seed, uint32_t stream) {
    int64_t n = nrows * cols;
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < n; ++e) {
        uint64_t gi = (uint64_t)(row0 * cols + e);
        float z = (float)ih12(seed, stream, gi) * (1.0f / 65536.0f);
        out[e] = sigma * z;
    }
}

/* 1 + jitter * z, for norm weight vectors (jitter 0 gives exact ones). */
void aw4s_one_plus_normal_f32(float* out, int64_t n, float jitter, uint64_t seed, uint32_t stream) {
    for (int64_t e = 0; e < n; ++e) {
        float z = (float)ih12(seed, stream, (uint64_t)e) * (1.0f / 65536.0f);
        out[e] = 1.0f + jitter * z;
    }
}

void aw4s_u32(uint32_t* out, int64_t i0, int64_t n, uint64_t seed, uint32_t stream) {
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < n; ++e) out[e] = aw4s_u32_at(seed, stream, (uint64_t)(i0 + e));
}

/* uniform floats in [0, 1): top 24 bits of a word times 2^-24 (exact) */
void aw4s_uniform_f32(float* out, int64_t i0, int64_t n, uint64_t seed, uint32_t stream) {
    for (int64_t e = 0; e < n; ++e)
        out[e] = (float)(aw4s_u32_at(seed, stream, (uint64_t)(i0 + e)) >> 8) * (1.0f / 16777216.0f);
}

/* token ids in [0, vocab): multiply-shift of a 32-bit word */
void aw4s_tokens(int32_t* out, int64_t i0, int64_t n, int32_t vocab, uint64_t seed, uint32_t stream) {
    for (int64_t e = 0; e < n; ++e)
        out[e] = (int32_t)(((uint64_t)aw4s_u32_at(seed, stream, (uint64_t)(i0 + e)) * (uint64_t)vocab) >> 32);
}

/* +1 / -1 from bit 31 of a word */
void aw4s_signs(int8_t* out, int64_t n, uint64_t seed, uint32_t stream) {
    for (int64_t e = 0; e < n; ++e)
        out[e] = (aw4s_u32_at(seed, stream, (uint64_t)e) >> 31) ? (int8_t)-1 : (int8_t)1;
}

/* Integer codes with a discretised-normal shape:
 *   c = clamp(floor((ih12 * spread256 + 2^23) / 2^24), -qmax, qmax)
 * i.e. round(z * spread256 / 256) computed in integers. */
void aw4s_codes_i8(int8_t* out, int64_t i0, int64_t n, int32_t spread256, int32_t qmax,
                   uint64_t seed, uint32_t stream) {
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < n; ++e) {
        int64_t v = (int64_t)ih12(seed, stream, (uint64_t)(i0 + e)) * spread256 + (1ll << 23);
        int64_t c = v >> 24;  /* arithmetic shift: floor */
        if (c > qmax) c = qmax;
        if (c < -qmax) c = -qmax;
        out[e] = (int8_t)c;
    }
}

/* fp16 bit patterns base_bits + (u32 >> 28) - 8: scales spread over 16 ulps */
void aw4s_scale_bits(uint16_t* out, int64_t i0, int64_t n, uint16_t base_bits, uint64_t seed,
                     uint32_t stream) {
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < n; ++e)
        out[e] = (uint16_t)(base_bits + (aw4s_u32_at(seed, stream, (uint64_t)(i0 + e)) >> 28) - 8u);
}

// Prefill on gfx950: a chunk of prompt tokens through every layer at once.
//
// Prefill is the step before decode (the pages time it apart from decode:
// page 3 "Qwen3.8-27B 實測", the prompt-processing figures of the NVFP4 vLLM
// and DGX Spark runs, and page 4's note that a 100K-token input takes about
// two minutes).  Every token computes what a decode step computes (the same
// fp16 inputs, fp32 accumulation, the same KV codec and GDN recurrence); what
// changes is that the weights are read once per chunk:
//   - W4 GEMM on the matrix cores with exact weights: one product per 32-value
//     group of exact codes against the fp16 inputs (exact products, fp32
//     sums), then the row's fp16 group scale applied in fp32, as the decode
//     GEMV does;
//   - Gated DeltaNet: the normalised q, k and the gates of all chunk tokens
//     first, then one workgroup per (v head, 16 state rows) runs the tokens in
//     order with its rows of S in registers;
//   - attention: the decode kernels (append, multi-token sweeps, combine) with
//     one sweep block per few tokens of the chunk.
#include "aw4_internal.h"

#include <algorithm>

namespace aw4 {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ float half_bits_to_float(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
// logistic function with the hardware reciprocal, as the decode GEMV epilogues
__device__ __forceinline__ float sigmoid_rcp(float v) { return __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }
// logistic function as the decode GDN kernel computes it
__device__ __forceinline__ float sigmoid_div(float v) { return 1.0f / (1.0f + __expf(-v)); }

__device__ __forceinline__ float wsum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float block_sum256(float v, float* red) {
    v = wsum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

// ------------------------------------------------------------------ W4 GEMM
// Y[m][n] = sum_k X[m][k] W[n][k] over M tokens: a workgroup of four waves
// covers 128 rows x 128 tokens, each wave 64 x 64 (4 x 4 blocks of 16 x 16).
// Stages of two 32-value groups: the token tile (fp16), the rows' code dwords
// and their scales are staged in LDS (double buffered; two register sets hold
// the next two stages, so a stage's loads have two stages of products to
// arrive in).  A operand: 16 rows' exact codes, lane (c, q) row c, values
// 8q..8q+7 of the group (one code dword, nibble slots [0,2,4,6,1,3,5,7]);
// B operand: 16 tokens, lane (c, q) token c, the same values.  D lane (c, q)
// holds rows 4q..4q+3 of token c, which take their rows' scales before they
// are added to the accumulators.
constexpr int kGBK = 64;            // K values per stage (two groups)
// LDS position of code dword d of row R: d ^ cswz(R) within the row's 8
// dwords.  A wave reads dword 4 g + q of rows r + c (c < 16) for one group g;
// unswizzled, 16 rows 32 bytes apart fill only 16 of the 32 banks (4-way
// conflicts); XOR with 0, 1, 4 or 5 by (R >> 2) & 3 spreads them over all 32
// (2-way, the least for 256 bytes).  The row's two 16-byte halves swap for
// 4 and 5, its dword pairs for 1 and 5.
__device__ __forceinline__ int cswz(int R) { return ((R >> 2) & 1) | (((R >> 3) & 1) << 2); }
constexpr int kGXP = kGBK + 8;      // padded LDS row of the token tile (halves)

// tile (rt, tt) of unit b: consecutive units go to the eight XCDs in turn, so
// the token tiles of one row tile run on one XCD back to back and its weights
// stay in that XCD's L2 (measured faster than giving each XCD one token tile
// and streaming the weights past it, and than XCD pairs taking two token
// tiles each, by 1-4%)
__device__ __forceinline__ void gemm_tile(int b, int ntt, int& rt, int& tt) {
    const int xcd = b & 7, kx = b >> 3;
    rt = 8 * (kx / ntt) + xcd;
    tt = kx % ntt;
}

// GEMM epilogue: lane (c, q) of wave (wr, wt) holds, in acc[rb][tb], rows
// n0 + 64 wr + 16 rb + 4q .. + 3 of token m0 + 64 wt + 16 tb + c
template <int EPI>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& a, const f4 (&acc)[4][4], int m0, int n0, int wr, int wt,
                                              int c, int q) {
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        const int m = m0 + 64 * wt + 16 * tb + c;
        if (m >= a.M) continue;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const int n = n0 + 64 * wr + 16 * rb + 4 * q;
            const f4 v = acc[rb][tb];
            if (EPI == EPI_SWIGLU) {
                // interleaved gate/up rows: (n, n + 1) and (n + 2, n + 3)
#pragma unroll
                for (int rr = 0; rr < 4; rr += 2)
                    if (n + rr + 1 < a.N)
                        a.hout[(int64_t)m * a.ldo + ((n + rr) >> 1)] = (_Float16)(v[rr] * sigmoid_rcp(v[rr]) * v[rr + 1]);
            } else {
                float* y = a.y + (int64_t)m * a.ldy + n;
                if (n + 3 < a.N && (a.ldy & 3) == 0) {
                    f4* y4 = (f4*)y;
                    *y4 = EPI == EPI_RESID ? *y4 + v : v;
                } else {
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        if (n + rr < a.N) y[rr] = EPI == EPI_RESID ? y[rr] + v[rr] : v[rr];
                }
            }
        }
    }
}

template <int EPI>
__global__ __launch_bounds__(256, 2) void k_gemm_w4(GemmArgs a) {
    __shared__ __align__(16) _Float16 xs[2][128][kGXP];
    __shared__ __align__(16) uint32_t cs[2][128][8];     // [row][group 0..1][dword 0..3]
    __shared__ __align__(16) uint16_t ss[2][2][128];     // [group][row]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, q = lane >> 4;
    const int wr = wave & 1, wt = wave >> 1;             // the wave's row and token halves
    const int G = a.K / 32, nstage = a.K / kGBK;

    // tiles in XCD order (gemm_tile).  Units past a.nfull are the splits of
    // the last tiles: split sp of tile a.nfull + x + 8 j (x < 8) is unit
    // a.nfull + x + 8 (j S + sp), so that the S splits of a tile run on its
    // XCD; split sp takes the stages [sp nstage / S, (sp + 1) nstage / S).
    const int ntt = (a.M + 127) / 128, nrt = (a.N + 127) / 128;
    int b = blockIdx.x, split = -1, st0 = 0, st1 = nstage;
    if (b >= a.nfull) {
        const int S = a.nsplit, j = b - a.nfull, grp = j >> 3;
        split = grp % S;
        b = a.nfull + (j & 7) + 8 * (grp / S);
        st0 = split * nstage / S;
        st1 = (split + 1) * nstage / S;
    }
    int rt, tt;
    gemm_tile(b, ntt, rt, tt);
    if (rt >= nrt) return;
    const int n0 = rt * 128, m0 = tt * 128;

    // staging: token chunk L = tid + 256 i (i < 4): token L / 8, halves 8 (L % 8);
    // codes and scales: row tid / 2, group tid % 2 of the stage
    const int srow = min(n0 + (tid >> 1), a.N - 1), sg = tid & 1;
    const uint4* cbase = (const uint4*)(a.codes + (int64_t)srow * G * 4) + sg;
    const uint16_t* sbase = a.scales + (int64_t)srow * G + sg;
    const _Float16* xbase[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int L = tid + 256 * i;
        xbase[i] = a.x + (int64_t)min(m0 + (L >> 3), a.M - 1) * a.ldx + 8 * (L & 7);
    }
    // two register sets for the stages in flight (plain named values: a
    // struct passed to the loaders by reference was kept on the stack, 176
    // bytes of scratch traffic per lane per stage pair)
    uint4 xa0, xa1, xa2, xa3, ca, xb0, xb1, xb2, xb3, cb;
    uint16_t sca, scb;
#define AW4_GLOAD(X0, X1, X2, X3, CW, SC, S)                       \
    {                                                              \
        const int k0_ = (S) * kGBK;                                \
        X0 = *(const uint4*)(xbase[0] + k0_);                      \
        X1 = *(const uint4*)(xbase[1] + k0_);                      \
        X2 = *(const uint4*)(xbase[2] + k0_);                      \
        X3 = *(const uint4*)(xbase[3] + k0_);                      \
        CW = cbase[2 * (S)];                                       \
        SC = sbase[2 * (S)];                                       \
    }
#define AW4_LSTORE(X0, X1, X2, X3, CW, SC, BUF)                    \
    {                                                              \
        *(uint4*)&xs[BUF][tid >> 3][8 * (tid & 7)] = X0;           \
        *(uint4*)&xs[BUF][(tid + 256) >> 3][8 * (tid & 7)] = X1;   \
        *(uint4*)&xs[BUF][(tid + 512) >> 3][8 * (tid & 7)] = X2;   \
        *(uint4*)&xs[BUF][(tid + 768) >> 3][8 * (tid & 7)] = X3;   \
        {                                                          \
            const int sw_ = cswz(tid >> 1);                        \
            *(uint4*)&cs[BUF][tid >> 1][4 * (sg ^ (sw_ >> 2))] =   \
                (sw_ & 1) ? uint4{CW.y, CW.x, CW.w, CW.z} : CW;    \
        }                                                          \
        ss[BUF][sg][tid >> 1] = SC;                                \
    }

    f4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
    const h2 off_lo = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 off_hi = {(_Float16)-72.0f, (_Float16)-72.0f};
    const f4 zero4 = {0.f, 0.f, 0.f, 0.f};

    // the fp16 exponent bits of the code slots, in a register: (w & mask) | it
    // is then one v_and_or_b32 (with both as literals it takes two)
    uint32_t k6400;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(k6400));

    // Eight (group, row block) steps per stage, software-pipelined: step t's
    // four products are issued before step t - 1's results take their
    // scales, so the FMAs wait on products issued a step earlier instead of
    // the ones just issued.
    auto compute = [&](int buf) {
        h8 bv[2][4];
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
                bv[g][tb] = *(const h8*)&xs[buf][64 * wt + 16 * tb + c][32 * g + 8 * q];
        f4 d[2][4];
        uint2 sv[2];
#pragma unroll
        for (int t = 0; t <= 8; ++t) {
            if (t < 8) {
                const int g = t >> 2, r = 64 * wr + 16 * (t & 3);
                // exact codes: lo slots 1024 + n - 1032, hi slots (1024 + 16 n) / 16 - 72
                const uint32_t w = cs[buf][r + c][(4 * g + q) ^ cswz(c)], w8 = w >> 8;
                const h2 p0 = as_h2((w & 0x000F000Fu) | k6400) + off_lo;
                const h2 p1 = __builtin_elementwise_fma(as_h2((w & 0x00F000F0u) | k6400), sixteenth, off_hi);
                const h2 p2 = as_h2((w8 & 0x000F000Fu) | k6400) + off_lo;
                const h2 p3 = __builtin_elementwise_fma(as_h2((w8 & 0x00F000F0u) | k6400), sixteenth, off_hi);
                const h8 av = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
                // fp16 scales of the four rows this lane's results belong to
                // (rows r + 4q .. r + 4q + 3), applied in fp32 after the product
                sv[t & 1] = *(const uint2*)&ss[buf][g][r + 4 * q];
#pragma unroll
                for (int tb = 0; tb < 4; ++tb)
                    d[t & 1][tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv[g][tb], zero4, 0, 0, 0);
            }
            if (t > 0) {
                const int u = t - 1, rb = u & 3;
                const uint2 s2 = sv[u & 1];
                const float s4[4] = {(float)as_h2(s2.x)[0], (float)as_h2(s2.x)[1], (float)as_h2(s2.y)[0],
                                     (float)as_h2(s2.y)[1]};
#pragma unroll
                for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        acc[rb][tb][rr] = __builtin_fmaf(s4[rr], d[u & 1][tb][rr], acc[rb][tb][rr]);
            }
        }
    };

    // unrolled by two so that the register sets keep fixed roles: in the first
    // half LDS buffer 0 holds stage s and sb stage s + 1, in the second half
    // buffer 1 holds stage s + 1 and sa stage s + 2.  Loads past the last
    // stage re-read it (the same straight-line loads every time, so the wait
    // counts stay exact); only the products of a missing odd stage are skipped.
    const int nst = st1 - st0;
    auto sidx = [&](int t) { return st0 + (t < nst ? t : nst - 1); };
    AW4_GLOAD(xa0, xa1, xa2, xa3, ca, sca, st0)
    AW4_GLOAD(xb0, xb1, xb2, xb3, cb, scb, sidx(1))
    AW4_LSTORE(xa0, xa1, xa2, xa3, ca, sca, 0)
    __syncthreads();
    for (int s = 0; s < nst; s += 2) {
        AW4_GLOAD(xa0, xa1, xa2, xa3, ca, sca, sidx(s + 2))
        compute(0);
        AW4_LSTORE(xb0, xb1, xb2, xb3, cb, scb, 1)
        __syncthreads();
        AW4_GLOAD(xb0, xb1, xb2, xb3, cb, scb, sidx(s + 3))
        if (s + 1 < nst) compute(1);
        AW4_LSTORE(xa0, xa1, xa2, xa3, ca, sca, 0)
        __syncthreads();
    }
#undef AW4_GLOAD
#undef AW4_LSTORE

    if (split >= 0) {
        // this split's partial tile, in the lanes' own order; k_gemm_combine
        // adds the splits and runs the epilogue after the launch
        f4* part = (f4*)a.part + ((int64_t)(b - a.nfull) * a.nsplit + split) * 4096 + wave * 1024 + lane;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) part[64 * (4 * rb + tb)] = acc[rb][tb];
        return;
    }
    gemm_epilogue<EPI>(a, acc, m0, n0, wr, wt, c, q);
}

// The split tiles of a k_gemm_w4 launch: one workgroup per tile, the same
// lane layout; the splits' partials added in split order, then the epilogue.
template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_combine(GemmArgs a) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane & 15, q = lane >> 4, wr = wave & 1, wt = wave >> 1;
    const int b = a.nfull + blockIdx.x, ntt = (a.M + 127) / 128, nrt = (a.N + 127) / 128;
    int rt, tt;
    gemm_tile(b, ntt, rt, tt);
    if (rt >= nrt) return;
    const f4* part = (const f4*)a.part + (int64_t)blockIdx.x * a.nsplit * 4096 + wave * 1024 + lane;
    f4 acc[4][4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) acc[rb][tb] = part[64 * (4 * rb + tb)];
    for (int sp = 1; sp < a.nsplit; ++sp)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) acc[rb][tb] += part[sp * 4096 + 64 * (4 * rb + tb)];
    gemm_epilogue<EPI>(a, acc, tt * 128, rt * 128, wr, wt, c, q);
}

// ------------------------------------------------------------------ row kernels
// token embedding rows of the tied int8 table, one workgroup per token
__global__ __launch_bounds__(256) void k_embed_rows(const int8_t* codes, const uint16_t* scales, int H,
                                                    const int32_t* tok, float* x) {
    const int t = blockIdx.x;
    const int64_t id = tok[t];
    for (int k = threadIdx.x; k < H; k += 256)
        x[(int64_t)t * H + k] = (float)codes[id * H + k] * half_bits_to_float(scales[id * (H / 32) + k / 32]);
}

// fp16(RMSNorm(x_t) * w), one workgroup per token (as the decode NORM prologue)
__global__ __launch_bounds__(256) void k_norm_rows(const float* x, const float* w, int K, float eps,
                                                   _Float16* out, int64_t ldo) {
    __shared__ float red[4];
    const float* xr = x + (int64_t)blockIdx.x * K;
    float ss = 0.f;
    for (int k = threadIdx.x; k < K; k += 256) ss += xr[k] * xr[k];
    ss = block_sum256(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)K + eps);
    _Float16* o = out + (int64_t)blockIdx.x * ldo;
    for (int k = threadIdx.x; k < K; k += 256) o[k] = (_Float16)(xr[k] * r * w[k]);
}

// GDN per token: q and k of every qk head L2-normalised, and the gates
// alpha = sigmoid(a + bias), beta = sigmoid(b) of every v head
__global__ __launch_bounds__(256) void k_gdn_prep(GdnPrefillArgs a) {
    const int t = blockIdx.x, D = a.d;
    const float* pr = a.proj + (int64_t)t * a.sproj;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    // one wave per (qk head, q or k) vector
    for (int v = wave; v < 2 * a.nqk; v += 4) {
        const int j = v >> 1, isk = v & 1;
        const float* src = pr + (int64_t)(isk ? a.nqk + j : j) * D;
        float ss = 0.f;
        for (int e = lane; e < D; e += 64) ss += src[e] * src[e];
        ss = wsum(ss);
        const float r = 1.0f / sqrtf(ss + a.eps);
        float* dst = (isk ? a.kn : a.qn) + ((int64_t)t * a.nqk + j) * D;
        for (int e = lane; e < D; e += 64) dst[e] = src[e] * r;
    }
    const float* av = pr + 2LL * a.nqk * D + 2LL * a.nv * D;
    for (int h = threadIdx.x; h < a.nv; h += 256) {
        a.ab[((int64_t)t * a.nv + h) * 2] = sigmoid_div(av[h] + a.a_bias[h]);
        a.ab[((int64_t)t * a.nv + h) * 2 + 1] = sigmoid_div(av[a.nv + h]);
    }
}

// GDN recurrence over the chunk's tokens in order: a workgroup owns ROWS rows
// of one v head's state, TPR = D / 8 lanes per row, eight state values per
// lane in registers; the next token's inputs are loaded while the current one
// is applied.
template <int D>
__global__ __launch_bounds__(256) void k_gdn_seq(GdnPrefillArgs a) {
    constexpr int EPT = 8;
    constexpr int TPR = D / EPT;
    constexpr int ROWS = 256 / TPR;
    // the chunk's inputs are staged in LDS TB tokens at a time (double
    // buffered, the next block's loads in flight while the current one runs):
    // with the inputs read from global memory one token ahead, every step
    // waited for a cache round trip
    constexpr int TB = 32;
    constexpr int KQ4 = TB * 2 * D / 4 / 256;   // float4 of k and q per thread per block
    constexpr int NVT = TB * ROWS / 256;         // v values per thread per block
    static_assert(KQ4 * 256 * 4 == TB * 2 * D && NVT * 256 == TB * ROWS, "staging shape");
    __shared__ __align__(16) float kq_s[2][TB][2][D];   // [buf][token][k, q][dim]
    __shared__ float v_s[2][TB][ROWS];
    __shared__ float ab_s[2][TB][2];
    const int tid = threadIdx.x;
    const int h = blockIdx.y;
    const int j = h / (a.nv / a.nqk);
    const int row0 = blockIdx.x * ROWS, rl = tid / TPR, r = row0 + rl;
    const int c0 = (tid % TPR) * EPT;
    float* Srow = a.S + ((int64_t)h * D + r) * D + c0;
    float s[8];
    {
        const float4 s0 = *(const float4*)Srow, s1 = *(const float4*)(Srow + 4);
        s[0] = s0.x; s[1] = s0.y; s[2] = s0.z; s[3] = s0.w;
        s[4] = s1.x; s[5] = s1.y; s[6] = s1.z; s[7] = s1.w;
    }
    // staged values in named registers (arrays captured by reference in a
    // lambda were kept on the stack)
    f4 rk[KQ4];
    float rv[NVT], rab = 0.f;
#define AW4_GDN_STAGE(BLK)                                                                                 \
    {                                                                                                      \
        /* tokens past the chunk re-read its last token (never used) */                                   \
        _Pragma("unroll") for (int i = 0; i < KQ4; ++i) {                                                  \
            const int idx = tid + 256 * i, tt = idx / (D / 2), rem = idx % (D / 2);                        \
            const int t = min((BLK) * TB + tt, a.T - 1);                                                   \
            const float* src = (rem < D / 4 ? a.kn : a.qn) + ((int64_t)t * a.nqk + j) * D + 4 * (rem % (D / 4)); \
            rk[i] = *(const f4*)src;                                                                       \
        }                                                                                                  \
        _Pragma("unroll") for (int i = 0; i < NVT; ++i) {                                                  \
            const int idx = tid + 256 * i, tt = idx / ROWS;                                                \
            const int t = min((BLK) * TB + tt, a.T - 1);                                                   \
            rv[i] = a.proj[(int64_t)t * a.sproj + 2LL * a.nqk * D + (int64_t)h * D + row0 + idx % ROWS];  \
        }                                                                                                  \
        if (tid < 2 * TB) {                                                                                \
            const int t = min((BLK) * TB + tid / 2, a.T - 1);                                              \
            rab = a.ab[((int64_t)t * a.nv + h) * 2 + (tid & 1)];                                           \
        }                                                                                                  \
    }
#define AW4_GDN_PUT(BUF)                                                                                   \
    {                                                                                                      \
        _Pragma("unroll") for (int i = 0; i < KQ4; ++i) ((f4*)&kq_s[BUF][0][0][0])[tid + 256 * i] = rk[i]; \
        _Pragma("unroll") for (int i = 0; i < NVT; ++i)(&v_s[BUF][0][0])[tid + 256 * i] = rv[i];          \
        if (tid < 2 * TB) (&ab_s[BUF][0][0])[tid] = rab;                                                   \
    }
    const int nblk = (a.T + TB - 1) / TB;
    AW4_GDN_STAGE(0)
    AW4_GDN_PUT(0)
    __syncthreads();
    for (int blk = 0; blk < nblk; ++blk) {
        const int buf = blk & 1;
        if (blk + 1 < nblk) AW4_GDN_STAGE(blk + 1)
        const int tn = min(TB, a.T - blk * TB);
        for (int tt = 0; tt < tn; ++tt) {
            const float4 k0 = *(const float4*)&kq_s[buf][tt][0][c0], k1 = *(const float4*)&kq_s[buf][tt][0][c0 + 4];
            const float4 q0 = *(const float4*)&kq_s[buf][tt][1][c0], q1 = *(const float4*)&kq_s[buf][tt][1][c0 + 4];
            const float v = v_s[buf][tt][rl], al = ab_s[buf][tt][0], be = ab_s[buf][tt][1];
            const float kk[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
            const float qq[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
            float u = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) u += s[e] * kk[e];
#pragma unroll
            for (int o = TPR / 2; o >= 1; o >>= 1) u += __shfl_xor(u, o, 64);
            const float delta = be * (v - al * u);
            float oo = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                s[e] = al * s[e] + delta * kk[e];
                oo += s[e] * qq[e];
            }
#pragma unroll
            for (int o = TPR / 2; o >= 1; o >>= 1) oo += __shfl_xor(oo, o, 64);
            if ((tid % TPR) == 0) a.o[(int64_t)(blk * TB + tt) * a.so + (int64_t)h * D + r] = oo;
        }
        if (blk + 1 < nblk) AW4_GDN_PUT(buf ^ 1)
        __syncthreads();
    }
#undef AW4_GDN_STAGE
#undef AW4_GDN_PUT
    *(float4*)Srow = make_float4(s[0], s[1], s[2], s[3]);
    *(float4*)(Srow + 4) = make_float4(s[4], s[5], s[6], s[7]);
}

// fp16(RMSNorm(o_h) * w * SiLU(z_h)) per (token, v head) of d values (as the
// decode GATED prologue); one workgroup per token, one wave per head in turn
__global__ __launch_bounds__(256) void k_gated_rows(GdnPrefillArgs a, const float* nw, _Float16* out, int64_t ldo) {
    const int t = blockIdx.x, D = a.d;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const float* o = a.o + (int64_t)t * a.so;
    const float* z = a.proj + (int64_t)t * a.sproj + 2LL * a.nqk * D + (int64_t)a.nv * D;
    for (int h = wave; h < a.nv; h += 4) {
        float ss = 0.f;
        for (int e = lane; e < D; e += 64) ss += o[h * D + e] * o[h * D + e];
        ss = wsum(ss);
        const float r = 1.0f / sqrtf(ss / (float)D + a.eps);
        for (int e = lane; e < D; e += 64) {
            const float zz = z[h * D + e];
            out[(int64_t)t * ldo + h * D + e] = (_Float16)(o[h * D + e] * r * nw[e] * (zz * sigmoid_rcp(zz)));
        }
    }
}

}  // namespace

// Tiles in rounds of the resident workgroups (P); when the last round is at
// most half full, its tiles are split S = P / tail ways along K (at most 8,
// at least one stage per split, at most a.part_slots partial tiles), so that
// it takes one round of 1/S-length units instead of a whole tile time on a
// partly idle chip (FFN gate/up at 1024 tokens: 2176 tiles on 512 slots,
// 4.25 rounds of work in 5); k_gemm_combine then adds the splits.
hipError_t launch_gemm_w4(int epi, const GemmArgs& a0, hipStream_t s) {
    if (a0.M < 1 || a0.N < 1 || a0.K % kGBK || a0.K < kGBK) return hipErrorInvalidValue;
    const void* fn = epi == EPI_STORE ? (const void*)k_gemm_w4<EPI_STORE>
                   : epi == EPI_RESID ? (const void*)k_gemm_w4<EPI_RESID>
                   : epi == EPI_SWIGLU ? (const void*)k_gemm_w4<EPI_SWIGLU> : nullptr;
    if (!fn) return hipErrorInvalidValue;
    GemmArgs a = a0;
    const int ntt = (a.M + 127) / 128, nrt = (a.N + 127) / 128;
    const int T = 8 * ntt * ((nrt + 7) / 8), nstage = a.K / kGBK;
    a.nfull = T;
    a.nsplit = 1;
    const int P = a.part ? resident_blocks(fn, 0) : 0;
    if (P >= 8 && P % 8 == 0 && T > P) {
        const int tail = T % P;
        int S = tail ? P / tail : 0;
        S = std::min(S, std::min(8, nstage));
        if (tail && (int64_t)tail * S > a.part_slots) S = a.part_slots / tail;
        if (S >= 2) {
            a.nfull = T - tail;
            a.nsplit = S;
        }
    }
    const dim3 grid(a.nfull + (T - a.nfull) * a.nsplit), block(256);
    if (epi == EPI_STORE) hipLaunchKernelGGL(k_gemm_w4<EPI_STORE>, grid, block, 0, s, a);
    else if (epi == EPI_RESID) hipLaunchKernelGGL(k_gemm_w4<EPI_RESID>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(k_gemm_w4<EPI_SWIGLU>, grid, block, 0, s, a);
    if (a.nsplit > 1) {
        const dim3 cg(T - a.nfull);
        if (epi == EPI_STORE) hipLaunchKernelGGL(k_gemm_combine<EPI_STORE>, cg, block, 0, s, a);
        else if (epi == EPI_RESID) hipLaunchKernelGGL(k_gemm_combine<EPI_RESID>, cg, block, 0, s, a);
        else hipLaunchKernelGGL(k_gemm_combine<EPI_SWIGLU>, cg, block, 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_embed_rows(const int8_t* codes, const uint16_t* scales, int H, const int32_t* tok, int T, float* x,
                             hipStream_t s) {
    hipLaunchKernelGGL(k_embed_rows, dim3(T), dim3(256), 0, s, codes, scales, H, tok, x);
    return hipGetLastError();
}

hipError_t launch_norm_rows(const float* x, const float* w, int K, float eps, int T, _Float16* out, int64_t ldo,
                            hipStream_t s) {
    hipLaunchKernelGGL(k_norm_rows, dim3(T), dim3(256), 0, s, x, w, K, eps, out, ldo);
    return hipGetLastError();
}

hipError_t launch_gdn_prefill(const GdnPrefillArgs& a, const float* gated_w, _Float16* out, int64_t ldo,
                              hipStream_t s) {
    if (a.T < 1 || a.nv % a.nqk) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_gdn_prep, dim3(a.T), dim3(256), 0, s, a);
    if (a.d == 128) hipLaunchKernelGGL(k_gdn_seq<128>, dim3(128 / 16, a.nv), dim3(256), 0, s, a);
    else if (a.d == 64) hipLaunchKernelGGL(k_gdn_seq<64>, dim3(64 / 32, a.nv), dim3(256), 0, s, a);
    else return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_gated_rows, dim3(a.T), dim3(256), 0, s, a, gated_w, out, ldo);
    return hipGetLastError();
}

}  // namespace aw4

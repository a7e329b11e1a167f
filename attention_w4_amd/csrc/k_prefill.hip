// Prefill on gfx950: a chunk of prompt tokens through every layer at once.
//
// Prefill is the step before decode (the pages time it apart from decode:
// page 3 "Qwen3.8-27B 實測", the prompt-processing figures of the NVFP4 vLLM
// and DGX Spark runs, and page 4's note that a 100K-token input takes about
// two minutes).  Every token computes what a decode step computes (the same
// fp16 inputs, fp32 accumulation, the same KV codec and GDN recurrence); what
// changes is that the weights are read once per chunk:
//   - W4 GEMM on the matrix cores with exact weights: the fp16 group scale s
//     splits into s_hi (its top 7 significant bits) and s_lo = s - s_hi (the
//     rest), code x s_hi and code x s_lo are both exact in fp16, and two
//     products per group accumulate in place in fp32;
//   - Gated DeltaNet: the normalised q, k and the gates of all chunk tokens
//     first, then one workgroup per (v head, 16 state rows) runs the tokens in
//     order with its rows of S in registers;
//   - attention: the decode kernels (append, multi-token sweeps, combine) with
//     one sweep block per few tokens of the chunk.
#include "aw4_internal.h"

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
// arrive in).  A operands: 16 rows' code x s_hi and code x s_lo, lane (c, q)
// row c, values 8q..8q+7 of the group (one code dword, nibble slots
// [0,2,4,6,1,3,5,7], and the row's scale);
// B operand: 16 tokens, lane (c, q) token c, the same values.  D lane (c, q)
// holds rows 4q..4q+3 of token c.
constexpr int kGBK = 64;            // K values per stage (two groups)
constexpr int kGXP = kGBK + 8;      // padded LDS row of the token tile (halves)

template <int EPI>
__global__ __launch_bounds__(256, 3) void k_gemm_w4(GemmArgs a) {
    __shared__ __align__(16) _Float16 xs[2][128][kGXP];
    __shared__ __align__(16) uint32_t cs[2][128][8];     // [row][group 0..1][dword 0..3]
    __shared__ __align__(16) uint16_t ss[2][2][128];     // [group][row]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, q = lane >> 4;
    const int wr = wave & 1, wt = wave >> 1;             // the wave's row and token halves
    const int G = a.K / 32, nstage = a.K / kGBK;

    // tiles in XCD order: consecutive workgroups go to the eight XCDs in turn,
    // so the token tiles of one row tile are given to one XCD back to back and
    // its weights stay in that XCD's L2 (measured faster than giving each XCD
    // one token tile and streaming the weights past it)
    const int ntt = (a.M + 127) / 128, nrt = (a.N + 127) / 128;
    const int b = blockIdx.x, xcd = b & 7, kx = b >> 3;
    const int rt = 8 * (kx / ntt) + xcd, tt = kx % ntt;
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
    struct Stage {
        uint4 x[4];
        uint4 cw;
        uint16_t sc;
    };
    auto gload = [&](Stage& st, int s) {
        const int k0 = s * kGBK;
#pragma unroll
        for (int i = 0; i < 4; ++i) st.x[i] = *(const uint4*)(xbase[i] + k0);
        st.cw = cbase[2 * s];
        st.sc = sbase[2 * s];
    };
    auto lstore = [&](const Stage& st, int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int L = tid + 256 * i;
            *(uint4*)&xs[buf][L >> 3][8 * (L & 7)] = st.x[i];
        }
        *(uint4*)&cs[buf][tid >> 1][4 * sg] = st.cw;
        ss[buf][sg][tid >> 1] = st.sc;
    };

    f4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
    const h2 off_lo = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 off_hi = {(_Float16)-72.0f, (_Float16)-72.0f};

    auto compute = [&](int buf) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            h8 bv[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
                bv[tb] = *(const h8*)&xs[buf][64 * wt + 16 * tb + c][32 * g + 8 * q];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int r = 64 * wr + 16 * rb;
                // exact codes: lo slots 1024 + n - 1032, hi slots (1024 + 16 n) / 16 - 72
                const uint32_t w = cs[buf][r + c][4 * g + q], w8 = w >> 8;
                const h2 p0 = as_h2((w & 0x000F000Fu) | 0x64006400u) + off_lo;
                const h2 p1 = __builtin_elementwise_fma(as_h2((w & 0x00F000F0u) | 0x64006400u), sixteenth, off_hi);
                const h2 p2 = as_h2((w8 & 0x000F000Fu) | 0x64006400u) + off_lo;
                const h2 p3 = __builtin_elementwise_fma(as_h2((w8 & 0x00F000F0u) | 0x64006400u), sixteenth, off_hi);
                // s = s_hi + s_lo, s_hi with 7 significant bits: |code| <= 8 keeps
                // both products exact in fp16 (s_lo may be subnormal)
                const uint16_t sb = ss[buf][g][r + c];
                const _Float16 shi = __builtin_bit_cast(_Float16, (uint16_t)(sb & 0xFFF0u));
                const _Float16 slo = __builtin_bit_cast(_Float16, sb) - shi;
                const h2 s2h = {shi, shi}, s2l = {slo, slo};
                const h2 a0 = p0 * s2h, a1 = p1 * s2h, a2 = p2 * s2h, a3 = p3 * s2h;
                const h2 b0 = p0 * s2l, b1 = p1 * s2l, b2 = p2 * s2l, b3 = p3 * s2l;
                const h8 ah = {a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
                const h8 al = {b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    acc[rb][tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bv[tb], acc[rb][tb], 0, 0, 0);
                    acc[rb][tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bv[tb], acc[rb][tb], 0, 0, 0);
                }
            }
        }
    };

    // unrolled by two so that the register sets keep fixed roles: in the first
    // half LDS buffer 0 holds stage s and sb stage s + 1, in the second half
    // buffer 1 holds stage s + 1 and sa stage s + 2.  Loads past the last
    // stage re-read it (the same straight-line loads every time, so the wait
    // counts stay exact); only the products of a missing odd stage are skipped.
    auto sidx = [&](int t) { return t < nstage ? t : nstage - 1; };
    Stage sa, sb;
    gload(sa, 0);
    gload(sb, sidx(1));
    lstore(sa, 0);
    __syncthreads();
    for (int s = 0; s < nstage; s += 2) {
        gload(sa, sidx(s + 2));
        compute(0);
        lstore(sb, 1);
        __syncthreads();
        gload(sb, sidx(s + 3));
        if (s + 1 < nstage) compute(1);
        lstore(sa, 0);
        __syncthreads();
    }

    // epilogue: lane (c, q) of block (rb, tb) holds rows 4q..4q+3 of token c
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
    const int h = blockIdx.y;
    const int j = h / (a.nv / a.nqk);
    const int r = blockIdx.x * ROWS + threadIdx.x / TPR;
    const int c0 = (threadIdx.x % TPR) * EPT;
    float* Srow = a.S + ((int64_t)h * D + r) * D + c0;
    float s[8];
    {
        const float4 s0 = *(const float4*)Srow, s1 = *(const float4*)(Srow + 4);
        s[0] = s0.x; s[1] = s0.y; s[2] = s0.z; s[3] = s0.w;
        s[4] = s1.x; s[5] = s1.y; s[6] = s1.z; s[7] = s1.w;
    }
    struct In {
        float4 k0, k1, q0, q1;
        float v, al, be;
    };
    auto load = [&](In& in, int t) {
        const float* kp = a.kn + ((int64_t)t * a.nqk + j) * D + c0;
        const float* qp = a.qn + ((int64_t)t * a.nqk + j) * D + c0;
        in.k0 = *(const float4*)kp;
        in.k1 = *(const float4*)(kp + 4);
        in.q0 = *(const float4*)qp;
        in.q1 = *(const float4*)(qp + 4);
        in.v = a.proj[(int64_t)t * a.sproj + 2LL * a.nqk * D + (int64_t)h * D + r];
        const float2 g = *(const float2*)(a.ab + ((int64_t)t * a.nv + h) * 2);
        in.al = g.x;
        in.be = g.y;
    };
    In cur, nxt;
    load(cur, 0);
    for (int t = 0; t < a.T; ++t) {
        if (t + 1 < a.T) load(nxt, t + 1);
        const float kk[8] = {cur.k0.x, cur.k0.y, cur.k0.z, cur.k0.w, cur.k1.x, cur.k1.y, cur.k1.z, cur.k1.w};
        const float qq[8] = {cur.q0.x, cur.q0.y, cur.q0.z, cur.q0.w, cur.q1.x, cur.q1.y, cur.q1.z, cur.q1.w};
        float u = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) u += s[e] * kk[e];
#pragma unroll
        for (int o = TPR / 2; o >= 1; o >>= 1) u += __shfl_xor(u, o, 64);
        const float delta = cur.be * (cur.v - cur.al * u);
        float oo = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            s[e] = cur.al * s[e] + delta * kk[e];
            oo += s[e] * qq[e];
        }
#pragma unroll
        for (int o = TPR / 2; o >= 1; o >>= 1) oo += __shfl_xor(oo, o, 64);
        if ((threadIdx.x % TPR) == 0) a.o[(int64_t)t * a.so + (int64_t)h * D + r] = oo;
        cur = nxt;
    }
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

hipError_t launch_gemm_w4(int epi, const GemmArgs& a, hipStream_t s) {
    if (a.M < 1 || a.N < 1 || a.K % kGBK || a.K < kGBK) return hipErrorInvalidValue;
    const int ntt = (a.M + 127) / 128, nrt = (a.N + 127) / 128;
    const dim3 grid(8 * ntt * ((nrt + 7) / 8)), block(256);
    if (epi == EPI_STORE) hipLaunchKernelGGL(k_gemm_w4<EPI_STORE>, grid, block, 0, s, a);
    else if (epi == EPI_RESID) hipLaunchKernelGGL(k_gemm_w4<EPI_RESID>, grid, block, 0, s, a);
    else if (epi == EPI_SWIGLU) hipLaunchKernelGGL(k_gemm_w4<EPI_SWIGLU>, grid, block, 0, s, a);
    else return hipErrorInvalidValue;
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

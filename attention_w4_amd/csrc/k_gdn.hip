// Gated DeltaNet recurrent step for one decode token on gfx950.
//
// The pages name the layer (page 5, bs178.com llamAmpere article,
// "为什么它真能这么快" point 一: 48 of the layers carry a Gated DeltaNet
// recurrent state instead of attention, and a kernel that gives each warp four
// state columns was worth 5-6%).  Per value head h with key head j:
//   q, k L2-normalised;  alpha = sigmoid(a + bias), beta = sigmoid(b)
//   S <- alpha S (I - beta k k^T) + beta v k^T = alpha S + beta (v - alpha S k) k^T
//   o = S q
// Rows of S are independent, so the work is split into (head, row-block)
// workgroups; each row of the fp32 state is read once and written once, the
// two row reductions (S k and S q) stay inside a group of lanes.
#include "aw4_internal.h"

namespace aw4 {
namespace {

__device__ __forceinline__ float sigmoidf_(float v) { return 1.0f / (1.0f + __expf(-v)); }

// D = head dim; TPR = threads per state row (D / 8 elements each)
template <int D>
__global__ __launch_bounds__(256) void k_gdn(GdnArgs a) {
    constexpr int EPT = 8;
    constexpr int TPR = D / EPT;            // 16 for D=128, 8 for D=64
    constexpr int ROWS = 256 / TPR;         // rows per block
    __shared__ float kq[2][D];
    __shared__ float red[2][8];
    const int h = blockIdx.y;
    const int j = h / (a.nv / a.nqk);
    const int row0 = blockIdx.x * ROWS;
    const int tid = threadIdx.x;
    // batch: sequence blockIdx.z's token, state and readout
    a.proj += blockIdx.z * a.sproj;
    a.S += blockIdx.z * a.sstride;
    a.o += blockIdx.z * a.so;

    const float* q = a.proj + (int64_t)j * D;
    const float* k = a.proj + (int64_t)a.nqk * D + (int64_t)j * D;
    const float* v = a.proj + 2LL * a.nqk * D + (int64_t)h * D;
    const float* av = a.proj + 2LL * a.nqk * D + 2LL * a.nv * D;
    const float* bv = av + a.nv;

    // k and q (cache-resident) are requested first and the state row after
    // them: vector loads retire in issue order, so the norm reductions can
    // start as soon as k and q arrive while the state's HBM reads are still in
    // flight.  Threads [0, D) take k, [D, 2D) take q; the others re-read k[0]
    // and drop it.
    const int kqi = tid < 2 * D ? tid : 0;
    float val = kqi < D ? k[kqi] : q[kqi - D];
    const int r = row0 + tid / TPR;
    const int c0 = (tid % TPR) * EPT;
    float* Srow = a.S + ((int64_t)h * D + r) * D + c0;
    const float4 s0 = *(const float4*)Srow;
    const float4 s1 = *(const float4*)(Srow + 4);
    const float vr = v[r];
    const float araw = av[h] + a.a_bias[h], braw = bv[h];
    asm volatile("" : "+v"(val));   // wait for k and q only
    if (tid >= 2 * D) val = 0.f;

    // L2 norms of k and q
    float ss = val * val;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
    const int wave = tid >> 6;
    if ((tid & 63) == 0) red[0][wave] = ss;
    __syncthreads();
    // waves [0, D/64) cover k, [D/64, 2D/64) cover q
    constexpr int WPV = D / 64;
    float ssk = 0.f, ssq = 0.f;
#pragma unroll
    for (int w = 0; w < WPV; ++w) { ssk += red[0][w]; ssq += red[0][WPV + w]; }
    if (tid < 2 * D) {
        const float r = 1.0f / sqrtf((tid < D ? ssk : ssq) + a.eps);
        kq[tid < D ? 0 : 1][tid < D ? tid : tid - D] = val * r;
    }
    __syncthreads();

    const float alpha = sigmoidf_(araw);
    const float beta = sigmoidf_(braw);

    float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    float u = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) u += s[e] * kq[0][c0 + e];
#pragma unroll
    for (int o = TPR / 2; o >= 1; o >>= 1) u += __shfl_xor(u, o, 64);
    const float delta = beta * (vr - alpha * u);
    float oo = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        s[e] = alpha * s[e] + delta * kq[0][c0 + e];
        oo += s[e] * kq[1][c0 + e];
    }
#pragma unroll
    for (int o = TPR / 2; o >= 1; o >>= 1) oo += __shfl_xor(oo, o, 64);
    *(float4*)Srow = make_float4(s[0], s[1], s[2], s[3]);
    *(float4*)(Srow + 4) = make_float4(s[4], s[5], s[6], s[7]);
    if ((tid % TPR) == 0) a.o[(int64_t)h * D + r] = oo;
}

}  // namespace

hipError_t launch_gdn(const GdnArgs& a, hipStream_t s) { return launch_gdn_batch(a, 1, s); }

hipError_t launch_gdn_batch(const GdnArgs& a, int B, hipStream_t s) {
    if (B < 1) return hipErrorInvalidValue;
    if (a.d == 128) {
        hipLaunchKernelGGL(k_gdn<128>, dim3(128 / 16, a.nv, B), dim3(256), 0, s, a);
    } else if (a.d == 64) {
        hipLaunchKernelGGL(k_gdn<64>, dim3(64 / 32, a.nv, B), dim3(256), 0, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace aw4

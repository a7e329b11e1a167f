// Draft verification (M = k + 1 <= 4 tokens in one pass) on gfx950: the Gated
// DeltaNet steps of the M tokens from the committed state S0 without writing
// it back, the replay that commits the accepted prefix, and the acceptance of
// draft tokens with probability min(1, p/q) followed by a draw from the
// renormalised residual max(0, p - q) or, when every draft is kept, a bonus
// draw from the last distribution (page 5, bs178.com llamAmpere article,
// "为什么它真能这么快" point 四: the draft head proposes, the target verifies
// them in parallel, and the accept rule leaves the output distribution equal to
// the target's; the old exact-match rule is the temperature-0 case).
#include "aw4_internal.h"
#include "block_scan.h"

namespace aw4 {
namespace {

__device__ __forceinline__ float sigmoidf_(float v) { return 1.0f / (1.0f + __expf(-v)); }

__device__ __forceinline__ float wsum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// M GDN steps of one (head, row block) from S0; o_m written, S untouched when
// commit_n < 0.  With commit_n >= 0 (the replay) the first n steps are applied
// and S written back, no readout.
template <int D>
__device__ __forceinline__ void gdn_multi_block(const GdnMultiArgs& a, int bx, int h) {
    constexpr int EPT = 8;
    constexpr int TPR = D / EPT;
    constexpr int ROWS = 256 / TPR;
    __shared__ float kq[4][2][D];
    __shared__ float red[4][2][4];
    const int j = h / (a.nv / a.nqk);
    const int row0 = bx * ROWS;
    const int tid = threadIdx.x, wave = tid >> 6;
    const int nsteps = a.replay ? *a.commit_n : a.M;

    // k and q of every step at once (threads [0, D) take k, [D, 2D) q): the
    // loads are issued together, and one barrier serves all the norms
    float val[4];
    {
        const int tq = tid < 2 * D ? tid : 0;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float* proj = a.proj + (m < nsteps ? m : 0) * a.sproj;
            const float v = tq < D ? proj[a.nqk * D + j * D + tq] : proj[j * D + tq - D];
            val[m] = m < nsteps && tid < 2 * D ? v : 0.f;
        }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        if (m >= nsteps) break;
        const float ss = wsum(val[m] * val[m]);
        if ((tid & 63) == 0) red[m][0][wave] = ss;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        if (m >= nsteps) break;
        constexpr int WPV = D / 64;
        float ssk = 0.f, ssq = 0.f;
#pragma unroll
        for (int w = 0; w < WPV; ++w) { ssk += red[m][0][w]; ssq += red[m][0][WPV + w]; }
        if (tid < 2 * D) {
            const float r = 1.0f / sqrtf((tid < D ? ssk : ssq) + a.eps);
            kq[m][tid < D ? 0 : 1][tid < D ? tid : tid - D] = val[m] * r;
        }
    }
    __syncthreads();

    const int r = row0 + tid / TPR;
    const int c0 = (tid % TPR) * EPT;
    float* Srow = a.S + ((int64_t)h * D + r) * D + c0;
    float4 s0 = *(const float4*)Srow;
    float4 s1 = *(const float4*)(Srow + 4);
    float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    for (int m = 0; m < nsteps; ++m) {
        const float* proj = a.proj + m * a.sproj;
        const float* av = proj + 2LL * a.nqk * D + 2LL * a.nv * D;
        const float alpha = sigmoidf_(av[h] + a.a_bias[h]);
        const float beta = sigmoidf_(av[a.nv + h]);
        const float vr = proj[2LL * a.nqk * D + (int64_t)h * D + r];
        float u = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) u += s[e] * kq[m][0][c0 + e];
#pragma unroll
        for (int o = TPR / 2; o >= 1; o >>= 1) u += __shfl_xor(u, o, 64);
        const float delta = beta * (vr - alpha * u);
        float oo = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            s[e] = alpha * s[e] + delta * kq[m][0][c0 + e];
            oo += s[e] * kq[m][1][c0 + e];
        }
        if (!a.replay) {
#pragma unroll
            for (int o = TPR / 2; o >= 1; o >>= 1) oo += __shfl_xor(oo, o, 64);
            if ((tid % TPR) == 0) a.o[m * a.so + (int64_t)h * D + r] = oo;
        }
    }
    if (a.replay && nsteps > 0) {
        *(float4*)Srow = make_float4(s[0], s[1], s[2], s[3]);
        *(float4*)(Srow + 4) = make_float4(s[4], s[5], s[6], s[7]);
    }
}

template <int D>
__global__ __launch_bounds__(256) void k_gdn_multi(GdnMultiArgs a) {
    gdn_multi_block<D>(a, blockIdx.x, blockIdx.y);
}

// The replay of every GDN layer in one launch (grid z: layer): the layers'
// replays are independent of each other once the accepted count is known.
template <int D>
__global__ __launch_bounds__(256) void k_gdn_replay(GdnReplayArgs r) {
    GdnMultiArgs a = r.a;
    const int l = blockIdx.z;
    a.proj = r.proj[l];
    a.a_bias = r.a_bias[l];
    a.S = r.S[l];
    gdn_multi_block<D>(a, blockIdx.x, blockIdx.y);
}

// ----------------------------------------------------------------- acceptance
// Per block of the vocabulary (kAccChunk entries), per distribution j:
//   z[j][b]  = sum exp((L_j - max_j) / T)                    (pass 1)
//   w[j][b]  = sum max(0, p_j - q_j) for j < k, sum p_k      (pass 2)
constexpr int kAccChunk = 2048;
constexpr int kAccMaxChunks = 1024;   // vocabularies up to 2M ids

__global__ __launch_bounds__(256) void k_acc_z(AcceptArgs a) {
    __shared__ float red[4];
    const int b = blockIdx.x, j = blockIdx.y;
    const float mx = a.ctl->vmax[j];
    const float* L = a.logits + (int64_t)j * a.V;
    const int v0 = b * kAccChunk, v1 = min(a.V, v0 + kAccChunk);
    float s = 0.f;
    for (int v = v0 + threadIdx.x; v < v1; v += 256) s += __expf((L[v] - mx) * a.inv_t);
    s = wsum(s);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) a.zpart[j * gridDim.x + b] = red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(256) void k_acc_zsum(AcceptArgs a, int nb) {
    // one block per distribution: fixed-order sum of the block partials
    __shared__ float red[4];
    const int j = blockIdx.x;
    float s = 0.f;
    for (int b = threadIdx.x; b < nb; b += 256) s += a.zpart[j * nb + b];
    s = wsum(s);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) a.ctl->vz[j] = red[0] + red[1] + red[2] + red[3];
}

__device__ __forceinline__ float resid_w(const AcceptArgs& a, int j, int v) {
    const float p = __expf((a.logits[(int64_t)j * a.V + v] - a.ctl->vmax[j]) * a.inv_t) / a.ctl->vz[j];
    if (j == a.k) return p;   // bonus distribution
    return fmaxf(0.f, p - a.q[(int64_t)j * a.V + v]);
}

__global__ __launch_bounds__(256) void k_acc_w(AcceptArgs a) {
    __shared__ float red[4];
    const int b = blockIdx.x, j = blockIdx.y;
    const int v0 = b * kAccChunk, v1 = min(a.V, v0 + kAccChunk);
    float s = 0.f;
    for (int v = v0 + threadIdx.x; v < v1; v += 256) s += resid_w(a, j, v);
    s = wsum(s);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) a.wpart[j * gridDim.x + b] = red[0] + red[1] + red[2] + red[3];
}

// Sequential decisions (one thread), then the draw: inverse CDF in index order
// over the chosen distribution, the chunk of the crossing from the chunk
// masses and the index inside it, both by a block-wide scan (block_scan.h).
__global__ __launch_bounds__(256) void k_acc_decide(AcceptArgs a, int nb) {
    __shared__ int s_choice;     // distribution to draw from, or -1 (greedy / none)
    __shared__ BlockScanLds sl;
    __shared__ float part[kAccMaxChunks];
    __shared__ float chunk[kAccChunk];
    __shared__ float s_before;
    Ctl* c = a.ctl;
    const int k = a.k, tid = threadIdx.x;
    if (tid == 0) {
        int n_acc = 0;
        int choice = -1;
        bool stop = false;
        for (int j = 0; j < k && !stop; ++j) {
            const int d = c->vtok[j + 1];
            if (a.greedy) {
                if (c->vargmax[j] == d) ++n_acc;
                else stop = true;
            } else {
                const float p = __expf((a.logits[(int64_t)j * a.V + d] - c->vmax[j]) * a.inv_t) / c->vz[j];
                const float qd = a.q[(int64_t)j * a.V + d];
                const float ratio = qd > 0.f ? p / qd : 0.f;
                if (c->vu[j] < fminf(1.f, ratio)) ++n_acc;
                else { stop = true; choice = j; }
            }
        }
        if (!stop && !a.greedy) choice = k;   // every draft kept: bonus draw
        for (int j = 0; j < n_acc; ++j) c->vout[j] = c->vtok[j + 1];
        c->vn_acc = n_acc;
        c->vn_out = n_acc + 1;
        c->vcommit = n_acc + 1;
        if (a.greedy) c->vout[n_acc] = c->vargmax[n_acc];
        s_choice = choice;
    }
    __syncthreads();
    const int choice = s_choice;
    if (choice < 0) return;
    const float mx = c->vmax[choice], inv_z = 1.0f / c->vz[choice];
    for (int b = tid; b < kAccMaxChunks; b += 256) part[b] = b < nb ? a.wpart[choice * nb + b] : 0.f;
    __syncthreads();
    float tot = block_sum_lds<kAccMaxChunks / 256>(part, nb, sl);
    // an all-zero residual falls back to p itself: chunk masses of p
    const bool use_p = !(tot > 0.f);
    if (use_p) {
        for (int b = tid; b < nb; b += 256) {
            const int v0 = b * kAccChunk, v1 = min(a.V, v0 + kAccChunk);
            float bs = 0.f;
            for (int v = v0; v < v1; ++v) bs += __expf((a.logits[(int64_t)choice * a.V + v] - mx) * a.inv_t) * inv_z;
            part[b] = bs;
        }
        __syncthreads();
        tot = block_sum_lds<kAccMaxChunks / 256>(part, nb, sl);
    }
    if (tid == 0) c->vresid_p = use_p ? 1 : 0;
    const float target = c->vu[k] * tot;
    const int blk0 = block_inverse_cdf<kAccMaxChunks / 256>(part, nb, 0.f, target, &s_before, sl);
    const int blk = blk0 < 0 ? nb - 1 : blk0;
    const float base = blk0 < 0 ? 0.f : s_before;
    __syncthreads();
    const int v0 = blk * kAccChunk, v1 = min(a.V, v0 + kAccChunk);
    for (int v = v0 + tid; v < v0 + kAccChunk; v += 256) {
        float w = 0.f;
        if (v < v1) {
            const float p = __expf((a.logits[(int64_t)choice * a.V + v] - mx) * a.inv_t) * inv_z;
            w = (use_p || choice == k) ? p : fmaxf(0.f, p - a.q[(int64_t)choice * a.V + v]);
        }
        chunk[v - v0] = w;
    }
    __syncthreads();
    const int pick = block_inverse_cdf<kAccChunk / 256>(chunk, v1 - v0, base, target, &s_before, sl);
    if (tid == 0) c->vout[c->vn_acc] = pick < 0 ? v0 : v0 + pick;
}

// per-distribution max and argmax from the head's block partials
__global__ __launch_bounds__(256) void k_acc_max(const float* pv, const int32_t* pi, int nb, Ctl* ctl) {
    __shared__ float sv[256];
    __shared__ int si[256];
    const int j = blockIdx.x;
    float b = -INFINITY;
    int bi = 0x7fffffff;
    for (int i = threadIdx.x; i < nb; i += 256) {
        const float v = pv[j * nb + i];
        const int ix = pi[j * nb + i];
        if (v > b || (v == b && ix < bi)) { b = v; bi = ix; }
    }
    sv[threadIdx.x] = b;
    si[threadIdx.x] = bi;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (threadIdx.x < s) {
            const float v = sv[threadIdx.x + s];
            const int ix = si[threadIdx.x + s];
            if (v > sv[threadIdx.x] || (v == sv[threadIdx.x] && ix < si[threadIdx.x])) {
                sv[threadIdx.x] = v;
                si[threadIdx.x] = ix;
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        ctl->vmax[j] = sv[0];
        ctl->vargmax[j] = si[0] == 0x7fffffff ? 0 : si[0];
    }
}

__global__ void k_commit_pos(Ctl* ctl) {
    ctl->pos += ctl->vcommit;
    ctl->token = ctl->vout[ctl->vn_out - 1];
}

}  // namespace

hipError_t launch_gdn_multi(const GdnMultiArgs& a, hipStream_t s) {
    if (a.M < 1 || a.M > 4) return hipErrorInvalidValue;
    if (a.d == 128) hipLaunchKernelGGL(k_gdn_multi<128>, dim3(128 / 16, a.nv), dim3(256), 0, s, a);
    else if (a.d == 64) hipLaunchKernelGGL(k_gdn_multi<64>, dim3(64 / 32, a.nv), dim3(256), 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_gdn_replay(const GdnReplayArgs& r, hipStream_t s) {
    const GdnMultiArgs& a = r.a;
    if (a.M < 1 || a.M > 4 || !a.replay || !a.commit_n || r.nlayers < 1 || r.nlayers > kMaxReplayLayers)
        return hipErrorInvalidValue;
    if (a.d == 128) hipLaunchKernelGGL(k_gdn_replay<128>, dim3(128 / 16, a.nv, r.nlayers), dim3(256), 0, s, r);
    else if (a.d == 64) hipLaunchKernelGGL(k_gdn_replay<64>, dim3(64 / 32, a.nv, r.nlayers), dim3(256), 0, s, r);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

int accept_blocks(int V) { return (V + kAccChunk - 1) / kAccChunk; }

hipError_t launch_accept(const AcceptArgs& a, const float* head_pv, const int32_t* head_pi, int head_nb,
                         hipStream_t s) {
    const int nb = accept_blocks(a.V);
    if (nb > kAccMaxChunks) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_acc_max, dim3(a.k + 1), dim3(256), 0, s, head_pv, head_pi, head_nb, a.ctl);
    if (!a.greedy) {
        hipLaunchKernelGGL(k_acc_z, dim3(nb, a.k + 1), dim3(256), 0, s, a);
        hipLaunchKernelGGL(k_acc_zsum, dim3(a.k + 1), dim3(256), 0, s, a, nb);
        hipLaunchKernelGGL(k_acc_w, dim3(nb, a.k + 1), dim3(256), 0, s, a);
    }
    hipLaunchKernelGGL(k_acc_decide, dim3(1), dim3(256), 0, s, a, nb);
    return hipGetLastError();
}

hipError_t launch_head_argmax_multi(const float* pv, const int32_t* pi, int nb, int M, Ctl* ctl, hipStream_t s) {
    if (M < 1 || M > 4) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_acc_max, dim3(M), dim3(256), 0, s, pv, pi, nb, ctl);
    return hipGetLastError();
}

hipError_t launch_commit_pos(Ctl* ctl, hipStream_t s) {
    hipLaunchKernelGGL(k_commit_pos, dim3(1), dim3(1), 0, s, ctl);
    return hipGetLastError();
}

}  // namespace aw4

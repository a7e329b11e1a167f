// The draft head's own kernels on gfx950: its input (the normalised embedding
// of the current token beside the normalised hidden state, in fp16) and the
// choice of a draft from the mapped scores.
//
// The pages' draft head (page 5, bs178.com llamAmpere article, "为什么它真能这么快"
// point 四) proposes three tokens from the model's own state and scores them
// only over a list of 65,536 ids; the target keeps the full vocabulary.  At
// temperature 0 a draft is the best mapped id (lowest id on ties); at T > 0 it
// is drawn from q = softmax(score / T) over the map by inverse CDF in ascending
// id order, and q, zero outside the map, is what the verify pass divides by.
// The block between input and scores runs on the W4 GEMV, attention and head
// kernels of the target.
#include "aw4_internal.h"

namespace aw4 {
namespace {

constexpr int kDraftChunk = 2048;   // map entries per block of the normaliser sums

__device__ __forceinline__ float wsum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

// one workgroup per entry m: RMSNorm of the dequantised table row of tok[m]
// and of h_m, each with its own weight, written side by side as fp16
__global__ __launch_bounds__(256) void k_draft_embed(DraftEmbedArgs a) {
    __shared__ float red[2][4];
    const int m = blockIdx.x, H = a.H;
    const int64_t tok = a.tok[m];
    const int8_t* cr = a.codes + tok * H;
    const uint16_t* sr = a.scales + tok * (H / 32);
    const float* h = a.h + (int64_t)m * a.sh;
    float se = 0.f, sh = 0.f;
    for (int k = threadIdx.x; k < H; k += 256) {
        const float e = (float)cr[k] * half_bits_to_float(sr[k >> 5]);
        const float v = h[k];
        se += e * e;
        sh += v * v;
    }
    se = wsum(se);
    sh = wsum(sh);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red[0][wave] = se;
        red[1][wave] = sh;
    }
    __syncthreads();
    se = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    sh = red[1][0] + red[1][1] + red[1][2] + red[1][3];
    const float re = 1.0f / sqrtf(se / (float)H + a.eps);
    const float rh = 1.0f / sqrtf(sh / (float)H + a.eps);
    _Float16* u = a.u + (int64_t)m * 2 * H;
    for (int k = threadIdx.x; k < H; k += 256) {
        const float e = (float)cr[k] * half_bits_to_float(sr[k >> 5]);
        u[k] = (_Float16)(e * re * a.nw_emb[k]);
        u[H + k] = (_Float16)(h[k] * rh * a.nw_hid[k]);
    }
}

// best mapped score and its index from the head's block partials (lowest index
// on ties); at temperature 0 that is the draft.  The first step of a call also
// commits its entries to the draft cache length.
__global__ __launch_bounds__(256) void k_dsel_max(DraftSelArgs a) {
    __shared__ float sv[256];
    __shared__ int si[256];
    float b = -INFINITY;
    int bi = 0x7fffffff;
    for (int i = threadIdx.x; i < a.nb; i += 256) {
        const float v = a.pv[i];
        const int ix = a.pi[i];
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
        Ctl* c = a.ctl;
        const int best = si[0] == 0x7fffffff ? 0 : si[0];
        c->dmax = sv[0];
        c->darg = best;
        if (a.greedy) c->dout[a.j] = a.map[best];
        if (a.commit) c->dpos += a.commit;
    }
}

__device__ __forceinline__ float dweight(const DraftSelArgs& a, int i) {
    return __expf((a.z[i] - a.ctl->dmax) * a.inv_t);
}

// per chunk of the map: sum of exp((z - max) / T)
__global__ __launch_bounds__(256) void k_dsel_z(DraftSelArgs a) {
    __shared__ float red[4];
    const int i0 = blockIdx.x * kDraftChunk, i1 = min(a.Vd, i0 + kDraftChunk);
    float s = 0.f;
    for (int i = i0 + threadIdx.x; i < i1; i += 256) s += dweight(a, i);
    s = wsum(s);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) a.zpart[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

// the normaliser (fixed-order sum of the chunks), then the draw: the chunk in
// which the running sum passes u Z, and the index inside it by a scan
__global__ __launch_bounds__(256) void k_dsel_draw(DraftSelArgs a, int nchunks) {
    __shared__ float s_target, s_base;
    __shared__ int s_chunk;
    __shared__ float w[kDraftChunk];
    Ctl* c = a.ctl;
    if (threadIdx.x == 0) {
        float Z = 0.f;
        for (int b = 0; b < nchunks; ++b) Z += a.zpart[b];
        c->dz = Z;
        const float target = c->du[a.j] * Z;
        float run = 0.f, base = 0.f;
        int blk = nchunks - 1;
        for (int b = 0; b < nchunks; ++b) {
            const float wb = a.zpart[b];
            if (run + wb > target && wb > 0.f) { blk = b; base = run; break; }
            run += wb;
            base = run;
        }
        s_target = target;
        s_base = base;
        s_chunk = blk;
    }
    __syncthreads();
    const int i0 = s_chunk * kDraftChunk, i1 = min(a.Vd, i0 + kDraftChunk);
    for (int i = i0 + threadIdx.x; i < i0 + kDraftChunk; i += 256) w[i - i0] = i < i1 ? dweight(a, i) : 0.f;
    __syncthreads();
    if (threadIdx.x == 0) {
        float run = s_base;
        int pick = -1, last_nz = -1;
        for (int i = i0; i < i1; ++i) {
            const float wi = w[i - i0];
            if (wi > 0.f) last_nz = i;
            run += wi;
            if (run > s_target && wi > 0.f) { pick = i; break; }
        }
        if (pick < 0) pick = last_nz >= 0 ? last_nz : i0;   // rounding at the very end of the mass
        c->darg = pick;
        c->dout[a.j] = a.map[pick];
    }
}

// q over the whole vocabulary: q[v] = exp((z - max) / T) / Z on mapped ids, else 0
__global__ __launch_bounds__(256) void k_dsel_q(DraftSelArgs a) {
    const float inv_z = 1.0f / a.ctl->dz;
    for (int v = blockIdx.x * 256 + threadIdx.x; v < a.V; v += gridDim.x * 256) {
        const int i = a.rmap[v];
        a.q[v] = i >= 0 ? dweight(a, i) * inv_z : 0.f;
    }
}

struct DraftIn {
    int32_t tok[4];
    float u[4];
};

__global__ void k_set_draft(Ctl* ctl, DraftIn in) {
    for (int i = 0; i < 4; ++i) {
        ctl->dtok[i] = in.tok[i];
        ctl->du[i] = in.u[i];
        ctl->dout[i] = 0;
    }
}

__global__ void k_set_dpos(Ctl* ctl, int32_t dpos) { ctl->dpos = dpos; }

}  // namespace

int draft_chunks(int Vd) { return (Vd + kDraftChunk - 1) / kDraftChunk; }

hipError_t launch_draft_embed(const DraftEmbedArgs& a, hipStream_t s) {
    if (a.M < 1 || a.M > 4 || a.H % 32) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_draft_embed, dim3(a.M), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_draft_select(const DraftSelArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(k_dsel_max, dim3(1), dim3(256), 0, s, a);
    if (!a.greedy) {
        const int nc = draft_chunks(a.Vd);
        hipLaunchKernelGGL(k_dsel_z, dim3(nc), dim3(256), 0, s, a);
        hipLaunchKernelGGL(k_dsel_draw, dim3(1), dim3(256), 0, s, a, nc);
        if (a.q) {
            int g = (a.V + 255) / 256;
            if (g > 2048) g = 2048;
            hipLaunchKernelGGL(k_dsel_q, dim3(g), dim3(256), 0, s, a);
        }
    }
    return hipGetLastError();
}

hipError_t launch_set_draft(Ctl* ctl, const int32_t* tok, const float* u, hipStream_t s) {
    DraftIn in;
    for (int i = 0; i < 4; ++i) {
        in.tok[i] = tok[i];
        in.u[i] = u[i];
    }
    hipLaunchKernelGGL(k_set_draft, dim3(1), dim3(1), 0, s, ctl, in);
    return hipGetLastError();
}

hipError_t launch_set_dpos(Ctl* ctl, int32_t dpos, hipStream_t s) {
    hipLaunchKernelGGL(k_set_dpos, dim3(1), dim3(1), 0, s, ctl, dpos);
    return hipGetLastError();
}

}  // namespace aw4

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
#include "block_scan.h"

namespace aw4 {
namespace {

constexpr int kDraftChunk = 2048;      // map entries per block of the normaliser sums
constexpr int kDraftMaxChunks = 1024;  // so up to 2M mapped ids

__device__ __forceinline__ float wsum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

// one workgroup per entry m: RMSNorm of the dequantised table row of tok[m]
// and of h_m, each with its own weight, written side by side as fp16.  Each
// thread holds its four-value slices in registers, all loaded up front.
constexpr int kEmbMaxPer = 8;   // hidden sizes up to 8192

__global__ __launch_bounds__(256) void k_draft_embed(DraftEmbedArgs a) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    __shared__ float red[2][4];
    const int m = blockIdx.x, H = a.H, n4 = H / 4;
    const int64_t tok = a.tok[m];
    const uint32_t* cr = (const uint32_t*)(a.codes + tok * H);
    const uint16_t* sr = a.scales + tok * (H / 32);
    const float4* h = (const float4*)(a.h + (int64_t)m * a.sh);
    float4 ev[kEmbMaxPer], hv[kEmbMaxPer];
    float se = 0.f, sh = 0.f;
#pragma unroll
    for (int i = 0; i < kEmbMaxPer; ++i) {
        const int q = threadIdx.x + 256 * i;
        if (q < n4) {
            const uint32_t c4 = cr[q];
            const float sc = half_bits_to_float(sr[q >> 3]);
            ev[i] = make_float4((float)(int8_t)(c4 & 0xff) * sc, (float)(int8_t)((c4 >> 8) & 0xff) * sc,
                                (float)(int8_t)((c4 >> 16) & 0xff) * sc, (float)(int8_t)(c4 >> 24) * sc);
            hv[i] = h[q];
        } else {
            ev[i] = hv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        se += ev[i].x * ev[i].x + ev[i].y * ev[i].y + ev[i].z * ev[i].z + ev[i].w * ev[i].w;
        sh += hv[i].x * hv[i].x + hv[i].y * hv[i].y + hv[i].z * hv[i].z + hv[i].w * hv[i].w;
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
    h4* ue = (h4*)(a.u + (int64_t)m * 2 * H);
    h4* uh = (h4*)(a.u + (int64_t)m * 2 * H + H);
    const float4* we = (const float4*)a.nw_emb;
    const float4* wh = (const float4*)a.nw_hid;
#pragma unroll
    for (int i = 0; i < kEmbMaxPer; ++i) {
        const int q = threadIdx.x + 256 * i;
        if (q < n4) {
            const float4 a4 = we[q], b4 = wh[q];
            ue[q] = h4{(_Float16)(ev[i].x * re * a4.x), (_Float16)(ev[i].y * re * a4.y),
                       (_Float16)(ev[i].z * re * a4.z), (_Float16)(ev[i].w * re * a4.w)};
            uh[q] = h4{(_Float16)(hv[i].x * rh * b4.x), (_Float16)(hv[i].y * rh * b4.y),
                       (_Float16)(hv[i].z * rh * b4.z), (_Float16)(hv[i].w * rh * b4.w)};
        }
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

// the normaliser (sum of the chunk sums), then the draw: the chunk in which
// the running sum passes u Z, and the index inside it, both by a block-wide
// scan (block_scan.h)
__global__ __launch_bounds__(256) void k_dsel_draw(DraftSelArgs a, int nchunks) {
    __shared__ BlockScanLds sl;
    __shared__ float part[kDraftMaxChunks];
    __shared__ float w[kDraftChunk];
    __shared__ float s_before;
    Ctl* c = a.ctl;
    for (int b = threadIdx.x; b < kDraftMaxChunks; b += 256) part[b] = b < nchunks ? a.zpart[b] : 0.f;
    __syncthreads();
    const float Z = block_sum_lds<kDraftMaxChunks / 256>(part, nchunks, sl);
    const float target = c->du[a.j] * Z;
    const int blk0 = block_inverse_cdf<kDraftMaxChunks / 256>(part, nchunks, 0.f, target, &s_before, sl);
    const int blk = blk0 < 0 ? 0 : blk0;   // the best entry's weight is 1, so some chunk is nonzero
    const float base = blk0 < 0 ? 0.f : s_before;
    __syncthreads();
    const int i0 = blk * kDraftChunk, i1 = min(a.Vd, i0 + kDraftChunk);
    for (int i = threadIdx.x; i < kDraftChunk; i += 256) w[i] = i0 + i < i1 ? dweight(a, i0 + i) : 0.f;
    __syncthreads();
    const int pick = block_inverse_cdf<kDraftChunk / 256>(w, i1 - i0, base, target, &s_before, sl);
    if (threadIdx.x == 0) {
        const int idx = pick < 0 ? i0 : i0 + pick;
        c->dz = Z;
        c->darg = idx;
        c->dout[a.j] = a.map[idx];
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
    if (a.M < 1 || a.H % 32 || a.H > 4 * 256 * kEmbMaxPer) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_draft_embed, dim3(a.M), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_draft_select(const DraftSelArgs& a, hipStream_t s) {
    if (draft_chunks(a.Vd) > kDraftMaxChunks) return hipErrorInvalidValue;
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

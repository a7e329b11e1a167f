// Gated attention for one decode token over the compressed KV cache (gfx950).
//
// Cache format (page 5, bs178.com llamAmpere article, "为什么它真能这么快"
// point 三: keys kept at 8 bits because errors in them misfile everything,
// values rotated and compressed to about 3 bits): keys int8 per 32 with an
// fp16 scale; values v' = H D v / sqrt(d) (Sylvester Hadamard H, random signs
// D) then 3-bit codes -3..3 per 32 with an fp16 scale.  The same passage says
// the old dequant path of that cache reached only ~10% of usable bandwidth;
// here the cache is streamed position-major per kv head by many workgroups.
//
// k_attn: grid (split, kv head).  Every workgroup that needs the current token
// encodes its K and V (quantise K; sign flip, fast Walsh-Hadamard transform,
// quantise V); split 0 appends them to the cache.  Each workgroup then runs an
// online softmax over its range of positions for the q heads that share the kv
// head, accumulating values in the rotated domain, and writes (acc, m, l).
// k_combine: per q head, merges the splits (log-sum-exp), undoes the rotation
// once (D H acc / sqrt(d)), applies the output gate sigmoid(g) and emits fp16.
#include "aw4_internal.h"

namespace aw4 {
namespace {

__device__ __forceinline__ float sigmoidf_(float v) { return 1.0f / (1.0f + __expf(-v)); }

// max over aligned 32-lane segments
__device__ __forceinline__ float seg32_max(float v) {
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ void split_range(int npos, int nsplit, int& pps, int& used) {
    int p = (npos + nsplit - 1) / nsplit;
    pps = p < 64 ? 64 : p;
    used = (npos + pps - 1) / pps;
}

// in-place Sylvester fast Walsh-Hadamard transform of v[0..D) by D/2 threads
template <int D>
__device__ void fwht(float* v) {
    for (int hh = 1; hh < D; hh <<= 1) {
        if (threadIdx.x < D / 2) {
            const int t = threadIdx.x;
            const int i = (t / hh) * 2 * hh + (t % hh);
            const float x = v[i], y = v[i + hh];
            v[i] = x + y;
            v[i + hh] = x - y;
        }
        __syncthreads();
    }
}

// DPP sum inside each 16-lane row (every lane of the row gets the row sum)
#define AW4_DPP_ADD(v, ctrl)                                                                        \
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, \
                                                               0xF, 0xF, true))
__device__ __forceinline__ float row16_sum(float v) {
    AW4_DPP_ADD(v, 0xB1);    // quad_perm [1,0,3,2]
    AW4_DPP_ADD(v, 0x4E);    // quad_perm [2,3,0,1]
    AW4_DPP_ADD(v, 0x141);   // row_half_mirror
    AW4_DPP_ADD(v, 0x140);   // row_mirror
    return v;
}

// merge online-softmax states (m, l, acc) b into a
__device__ __forceinline__ float merge_scale(float& m, float mb, float& fa) {
    const float M = fmaxf(m, mb);
    fa = m == -INFINITY ? 0.f : __expf(m - M);
    const float fb = mb == -INFINITY ? 0.f : __expf(mb - M);
    m = M;
    return fb;
}

// Lane layout: a 16-lane row of a wave owns one cached position at a time,
// lane j of the row holds dims [DL*j, DL*j + DL) (DL = D/16).  The 16 rows of a
// workgroup (4 waves x 4 rows) walk the split's positions round robin, two
// positions per row in flight; each keeps its own online softmax state for the
// G query heads; rows and waves are merged at the end.
template <int D, int G>
__global__ __launch_bounds__(256) void k_attn(AttnArgs a) {
    constexpr int NG = D / 32;    // scale groups
    constexpr int DL = D / 16;    // dims per lane: 16 (D=256) or 4 (D=64)
    __shared__ float qs[G][D];
    __shared__ float vt[D];
    __shared__ int8_t kcur[D];
    __shared__ int8_t vcur[D];
    __shared__ float kscur[NG], vscur[NG];
    __shared__ uint16_t ksb[NG], vsb[NG];
    __shared__ float mm[4][G], ll[4][G];
    __shared__ float aa[4][G][D];

    const int split = blockIdx.x, j = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int row = lane >> 4, jl = lane & 15;
    const int pos = a.ctl->pos + a.pos_offset;
    const int npos = pos + 1;
    int pps, used;
    split_range(npos, a.nsplit, pps, used);
    if (split >= used) return;
    const int t0 = split * pps;
    const int t1 = min(npos, t0 + pps);
    const bool has_cur = (t1 == npos);
    const int64_t hbase = (int64_t)j * a.max_ctx;

    // queries of the G heads sharing kv head j, pre-scaled by 1/sqrt(D)
    const float qscale = 1.0f / sqrtf((float)D);
    {
        constexpr int N4 = G * D / 4;
        const float4* src = (const float4*)(a.proj + (int64_t)(j * G) * D);
#pragma unroll
        for (int i = 0; i < (N4 + 255) / 256; ++i) {
            const int idx = tid + 256 * i;
            if (idx < N4) {
                float4 q = src[idx];
                float* dst = &qs[0][0] + 4 * idx;
                dst[0] = q.x * qscale;
                dst[1] = q.y * qscale;
                dst[2] = q.z * qscale;
                dst[3] = q.w * qscale;
            }
        }
    }

    if (split == 0 || has_cur) {
        const float* kp = a.proj + 2LL * a.nq * D + (int64_t)j * D;
        const float* vp = kp + (int64_t)a.nkv * D;
        // K: int8 per 32
        {
            const float kv = tid < D ? kp[tid] : 0.f;
            const float am = seg32_max(fabsf(kv));
            const _Float16 sh = (_Float16)(am / 127.0f);
            const float sc = (float)sh;
            float c = sc == 0.f ? 0.f : rintf(kv / sc);
            c = fminf(fmaxf(c, -127.f), 127.f);
            if (tid < D) {
                kcur[tid] = (int8_t)c;
                if ((tid & 31) == 0) { kscur[tid >> 5] = sc; ksb[tid >> 5] = __builtin_bit_cast(uint16_t, sh); }
                vt[tid] = vp[tid] * a.signs[tid];
            }
        }
        __syncthreads();
        fwht<D>(vt);
        {
            const float vr = tid < D ? vt[tid] * qscale : 0.f;   // 1/sqrt(D): exact power of two here
            const float am = seg32_max(fabsf(vr));
            const _Float16 sh = (_Float16)(am / 3.0f);
            const float sc = (float)sh;
            float c = sc == 0.f ? 0.f : rintf(vr / sc);
            c = fminf(fmaxf(c, -3.f), 3.f);
            if (tid < D) {
                vcur[tid] = (int8_t)c;
                if ((tid & 31) == 0) { vscur[tid >> 5] = sc; vsb[tid >> 5] = __builtin_bit_cast(uint16_t, sh); }
            }
        }
        __syncthreads();
        if (split == 0) {
            const int64_t prow = hbase + pos;
            if (tid < D) a.kc[prow * D + tid] = kcur[tid];
            if (tid < NG) {
                a.ks[prow * NG + tid] = ksb[tid];
                a.vs[prow * NG + tid] = vsb[tid];
                uint32_t w[3] = {0u, 0u, 0u};
                for (int i = 0; i < 32; ++i) {
                    const uint32_t n = (uint32_t)(vcur[tid * 32 + i] + 4) & 7u;
                    const int bit = 3 * i, wi = bit >> 5, off = bit & 31;
                    w[wi] |= n << off;
                    if (off > 29) w[wi + 1] |= n >> (32 - off);
                }
                uint32_t* dst = a.vc + (prow * NG + tid) * 3;
                dst[0] = w[0];
                dst[1] = w[1];
                dst[2] = w[2];
            }
        }
    }
    __syncthreads();

    // this lane's query slices
    const int e0 = jl * DL;
    const int grp = e0 >> 5;
    float q[G][DL];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < DL; ++e) q[g][e] = qs[g][e0 + e];

    float m[G], l[G], acc[G][DL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < DL; ++e) acc[g][e] = 0.f;
    }
    // 3-bit fields of this lane's dims: group grp, values (e0 & 31) .. +DL-1
    const int bit0 = 3 * (e0 & 31);
    const int wi = bit0 >> 5, woff = bit0 & 31;
    const int rg = wave * 4 + row;   // row-group 0..15

    // Raw cache words of one position for this lane; dequantised at use so
    // that the loads of a whole batch stay in flight together (the current
    // token comes from the LDS copy: split 0 may still be writing its entry).
    struct Raw {
        uint32_t k[DL / 4];
        uint32_t vlo, vhi;
        uint16_t ks, vs;
        bool cur;
    };
    auto load_raw = [&](int t, Raw& r) {
        r.cur = (t == pos);
        if (r.cur) return;
        const int64_t prow = hbase + t;
        r.ks = a.ks[prow * NG + grp];
        r.vs = a.vs[prow * NG + grp];
        const int8_t* kr = a.kc + prow * D + e0;
        if (DL == 16) {
            const uint4 kw = *(const uint4*)kr;
            r.k[0] = kw.x; r.k[1] = kw.y; r.k[2] = kw.z; r.k[3] = kw.w;
        } else {
            r.k[0] = *(const uint32_t*)kr;
        }
        const uint32_t* vg = a.vc + (prow * NG + grp) * 3;
        r.vlo = vg[wi];
        r.vhi = wi < 2 ? vg[wi + 1] : 0u;
    };
    auto update = [&](const Raw& r) {
        float kf[DL], vf[DL];
        if (r.cur) {
#pragma unroll
            for (int e = 0; e < DL; ++e) {
                kf[e] = (float)kcur[e0 + e] * kscur[grp];
                vf[e] = (float)vcur[e0 + e] * vscur[grp];
            }
        } else {
            const float ksc = (float)__builtin_bit_cast(_Float16, r.ks);
            const float vsc = (float)__builtin_bit_cast(_Float16, r.vs);
#pragma unroll
            for (int e = 0; e < DL; ++e) kf[e] = (float)(int8_t)(r.k[e >> 2] >> (8 * (e & 3))) * ksc;
            const uint64_t bits = (((uint64_t)r.vhi << 32) | r.vlo) >> woff;
#pragma unroll
            for (int e = 0; e < DL; ++e) vf[e] = (float)((int)((bits >> (3 * e)) & 7u) - 4) * vsc;
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float p = 0.f;
#pragma unroll
            for (int e = 0; e < DL; ++e) p += q[g][e] * kf[e];
            const float sc = row16_sum(p);
            const float mn = fmaxf(m[g], sc);
            const float corr = __expf(m[g] - mn);
            const float pe = __expf(sc - mn);
            l[g] = l[g] * corr + pe;
#pragma unroll
            for (int e = 0; e < DL; ++e) acc[g][e] = acc[g][e] * corr + pe * vf[e];
            m[g] = mn;
        }
    };
    // positions t0 + rg + 16 k, in batches of NB per row-group with the next
    // batch's loads issued before the current one is used; a wave runs while any
    // of its rows has work (rows without skip, all lanes of a row agree)
    constexpr int NB = 4;
    Raw ra[NB] = {}, rn[NB] = {};
    int t = t0 + rg;
#pragma unroll
    for (int b = 0; b < NB; ++b)
        if (t + 16 * b < t1) load_raw(t + 16 * b, ra[b]);
    for (; t - row < t1; t += 16 * NB) {
        const int tn = t + 16 * NB;
        if (tn - row < t1) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if (tn + 16 * b < t1) load_raw(tn + 16 * b, rn[b]);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
            if (t + 16 * b < t1) update(ra[b]);
#pragma unroll
        for (int b = 0; b < NB; ++b) ra[b] = rn[b];
    }

    // merge the four rows of each wave (lanes jl, jl+16, jl+32, jl+48 hold the same dims)
#pragma unroll
    for (int sh = 16; sh <= 32; sh <<= 1) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float mb = __shfl_xor(m[g], sh, 64);
            const float lb = __shfl_xor(l[g], sh, 64);
            float fa;
            const float fb = merge_scale(m[g], mb, fa);
            l[g] = l[g] * fa + lb * fb;
#pragma unroll
            for (int e = 0; e < DL; ++e) acc[g][e] = acc[g][e] * fa + __shfl_xor(acc[g][e], sh, 64) * fb;
        }
    }
    if (row == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (jl == 0) { mm[wave][g] = m[g]; ll[wave][g] = l[g]; }
#pragma unroll
            for (int e = 0; e < DL; ++e) aa[wave][g][e0 + e] = acc[g][e];
        }
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += 256) {
        const int g = idx / D, e = idx % D;
        const float M = fmaxf(fmaxf(mm[0][g], mm[1][g]), fmaxf(mm[2][g], mm[3][g]));
        float L = 0.f, A = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float f = mm[w][g] == -INFINITY ? 0.f : __expf(mm[w][g] - M);
                L += ll[w][g] * f;
                A += aa[w][g][e] * f;
            }
        }
        float* dst = a.part + ((int64_t)(j * G + g) * a.nsplit + split) * (D + 2);
        dst[e] = A;
        if (e == 0) { dst[D] = M; dst[D + 1] = L; }
    }
}

template <int D>
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
    __shared__ float v[D];
    __shared__ float wsum[256];
    __shared__ float red[8];
    const int i = blockIdx.x, tid = threadIdx.x;
    const int pos = a.ctl->pos + a.pos_offset;
    int pps, used;
    split_range(pos + 1, a.nsplit, pps, used);
    const float* base = a.part + (int64_t)i * a.nsplit * (D + 2);
    // split weights exp(m_s - M) and the normaliser, one split per thread
    float ms = -INFINITY, ls = 0.f;
    if (tid < used) {
        ms = base[(int64_t)tid * (D + 2) + D];
        ls = base[(int64_t)tid * (D + 2) + D + 1];
    }
    float M = ms;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    if ((tid & 63) == 0) red[tid >> 6] = M;
    __syncthreads();
    M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float w = (tid < used && ms != -INFINITY) ? __expf(ms - M) : 0.f;
    wsum[tid] = w;
    float L = w * ls;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o, 64);
    __syncthreads();
    if ((tid & 63) == 0) red[4 + (tid >> 6)] = L;
    __syncthreads();
    L = red[4] + red[5] + red[6] + red[7];
    if (tid < D) {
        float A = 0.f;
        int s = 0;
        for (; s + 4 <= used; s += 4) {
            const float p0 = base[(int64_t)(s + 0) * (D + 2) + tid];
            const float p1 = base[(int64_t)(s + 1) * (D + 2) + tid];
            const float p2 = base[(int64_t)(s + 2) * (D + 2) + tid];
            const float p3 = base[(int64_t)(s + 3) * (D + 2) + tid];
            A += p0 * wsum[s] + p1 * wsum[s + 1] + p2 * wsum[s + 2] + p3 * wsum[s + 3];
        }
        for (; s < used; ++s) A += base[(int64_t)s * (D + 2) + tid] * wsum[s];
        v[tid] = A / L;
    }
    __syncthreads();
    fwht<D>(v);
    if (tid < D) {
        const float o = v[tid] * (1.0f / sqrtf((float)D)) * a.signs[tid];
        const float g = a.proj[(int64_t)a.nq * D + (int64_t)i * D + tid];
        a.out[(int64_t)i * D + tid] = (_Float16)(o * sigmoidf_(g));
    }
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
    const int G = a.nq / a.nkv;
    const dim3 grid(a.nsplit, a.nkv), block(256);
#define AW4_ATTN_CASE(DD, GG)                                                   \
    if (a.d == DD && G == GG) {                                                 \
        hipLaunchKernelGGL((k_attn<DD, GG>), grid, block, 0, s, a);             \
        return hipGetLastError();                                               \
    }
    AW4_ATTN_CASE(256, 6)
    AW4_ATTN_CASE(256, 4)
    AW4_ATTN_CASE(256, 8)
    AW4_ATTN_CASE(256, 2)
    AW4_ATTN_CASE(256, 1)
    AW4_ATTN_CASE(64, 4)
    AW4_ATTN_CASE(64, 2)
    AW4_ATTN_CASE(64, 1)
    AW4_ATTN_CASE(64, 6)
    AW4_ATTN_CASE(64, 8)
#undef AW4_ATTN_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
    if (a.nsplit > 256) return hipErrorInvalidValue;
    if (a.d == 256) hipLaunchKernelGGL(k_combine<256>, dim3(a.nq), dim3(256), 0, s, a);
    else if (a.d == 64) hipLaunchKernelGGL(k_combine<64>, dim3(a.nq), dim3(256), 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace aw4

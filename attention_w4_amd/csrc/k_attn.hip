// Gated attention for one decode token over the compressed KV cache (gfx950).
//
// Cache format (page 5, bs178.com llamAmpere article, "为什么它真能这么快"
// point 三: keys kept at 8 bits because errors in them misfile everything,
// values rotated and compressed to about 3 bits): keys int8 per 32 with an
// fp16 scale; values v' = H D v / sqrt(d) (Sylvester Hadamard H, random signs
// D) then 3-bit codes -3..3 per 32 with an fp16 scale.  The same passage says
// the old dequant path of that cache reached only ~10% of usable bandwidth;
// here the cache is streamed position-major per kv head by many workgroups and
// both products run on the matrix cores.
//
// Physical layout of one cached position (kv head j, position t):
//   key row, D bytes of code + 128: logical dim d = 32 g + 8 q + e (scale
//     group g, lane quarter q, e < 8) sits at byte 8 (D/32) q + 8 g + e, so the
//     8 keys a lane feeds to one 16x16x32 MFMA for each group are contiguous;
//   value record, 3 D / 8 bytes as 32-bit words: code + 4 of logical dim d in
//     bits 3 ((D/16) (d % 16) + d / 16) .. +2, so lane c of a 16x16x16 MFMA
//     finds the dims c, c + 16, c + 32, ... it needs as one 3 D / 16-bit field;
//   key and value scales: D/32 fp16 each, by group.
//
// k_attn: grid (split, kv head), 8 waves.  The workgroup whose range ends at
// the current token encodes its K and V (quantise K; sign flip, fast
// Walsh-Hadamard transform, quantise V) and appends them before anything reads
// the range.  Each wave takes 16-position tiles: scores S^T (16 positions x 16
// query-head slots) = sum over groups of key scale x (K_g Q_g^T), on
// 16x16x32 f16 MFMAs with exact int8 keys and q split into fp16 hi + lo parts;
// an online softmax per head; then O^T += V^T P'^T on 16x16x16 f16 MFMAs with
// exact codes and the value scale folded into P' (fp16 hi + lo again).  The
// score layout a lane holds (one head, four positions) is the B-operand layout
// of the second product, so P never leaves registers.  Waves merge through
// LDS; each split writes (acc, m, l) per query head.
// k_combine: per q head, merges the splits (log-sum-exp), undoes the rotation
// once (D H acc / sqrt(d)), applies the output gate sigmoid(g) and emits fp16.
#include "aw4_internal.h"

namespace aw4 {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;                    // waves per attention workgroup
constexpr int kTile = 16;                    // positions per wave tile; split lengths are multiples

__device__ __forceinline__ float sigmoidf_(float v) { return 1.0f / (1.0f + __expf(-v)); }

__device__ __forceinline__ void split_range(int npos, int nsplit, int& pps, int& used) {
    const int p = (npos + nsplit - 1) / nsplit;
    pps = (p + kTile - 1) / kTile * kTile;
    used = (npos + pps - 1) / pps;
}

template <int D>
__device__ __forceinline__ int k_byte(int d) {
    return 8 * (D / 32) * ((d & 31) >> 3) + 8 * (d >> 5) + (d & 7);
}

// Cache formats.  0: keys int8, values rotated then 3-bit codes -3..3 (field
// code + 4).  1 (q4_0: page 3 "Qwen3.8-27B 實測", section "RTX 5090 32GB", and
// page 4, jdon.com, on 262K contexts): keys and values 4-bit codes -7..7 per 32
// with an fp16 scale, values not rotated; a key row holds, per lane quarter q,
// one dword per scale group g (dword q NG + g) whose nibbles (code + 8) carry
// dims 32 g + 8 q + e in the slot order [0,2,4,6,1,3,5,7]; value fields are
// 4-bit (code + 8).  2: keys int8; values rotated, then the index of the
// nearest level of the 8-level Lloyd-Max Gaussian codebook, stored as a 3-bit
// sign (bit 2, set for the four negative levels) and magnitude (bits 0-1) field.
template <int FMT>
struct KvFmt {
    static constexpr int KB = FMT == 1 ? 4 : 8;       // key bits
    static constexpr int FB = FMT == 1 ? 4 : 3;       // value field bits
    static constexpr bool ROT = FMT != 1;             // values cached in the rotated domain
    static constexpr int KQMAX = FMT == 1 ? 7 : 127;
};

// Lloyd-Max codebook magnitudes (J. Max 1960, 8 levels for a unit Gaussian) as
// fp16: 0.2451, 0.7560, 1.3440, 2.1520, in the byte order a v_perm_b32 table
// needs (magnitude m at bytes 2 m, 2 m + 1 of the 8-byte pair hi:lo)
__device__ __forceinline__ void lm_table(uint32_t& lo, uint32_t& hi) {
    const _Float16 m0 = (_Float16)0.2451f, m1 = (_Float16)0.7560f, m2 = (_Float16)1.3440f, m3 = (_Float16)2.1520f;
    lo = (uint32_t)__builtin_bit_cast(uint16_t, m0) | ((uint32_t)__builtin_bit_cast(uint16_t, m1) << 16);
    hi = (uint32_t)__builtin_bit_cast(uint16_t, m2) | ((uint32_t)__builtin_bit_cast(uint16_t, m3) << 16);
}

// two sign-magnitude codebook fields (bits 0-2 and 16-18 of x) -> the two fp16 levels
__device__ __forceinline__ h2 lm_pair(uint32_t x, uint32_t tlo, uint32_t thi) {
    const uint32_t mag = x & 0x00030003u;
    const uint32_t sel = mag * 0x0202u + 0x01000100u;   // 2 m and 2 m + 1 in each half
    const uint32_t v = __builtin_amdgcn_perm(thi, tlo, sel);
    return __builtin_bit_cast(h2, v ^ ((x & 0x00040004u) << 13));
}

// eight 4-bit key fields of one dword (slot order [0,2,4,6,1,3,5,7], nibble =
// code + 8) -> the eight exact fp16 codes
__device__ __forceinline__ h8 nib8_to_h8(uint32_t w) {
    const h2 off_lo = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 off_hi = {(_Float16)-72.0f, (_Float16)-72.0f};
    const uint32_t w8 = w >> 8;
    const h2 p0 = __builtin_bit_cast(h2, (w & 0x000F000Fu) | 0x64006400u) + off_lo;
    const h2 p1 = __builtin_elementwise_fma(__builtin_bit_cast(h2, (w & 0x00F000F0u) | 0x64006400u), sixteenth, off_hi);
    const h2 p2 = __builtin_bit_cast(h2, (w8 & 0x000F000Fu) | 0x64006400u) + off_lo;
    const h2 p3 = __builtin_elementwise_fma(__builtin_bit_cast(h2, (w8 & 0x00F000F0u) | 0x64006400u), sixteenth, off_hi);
    const h8 r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    return r;
}

// eight offset-binary bytes u = b + 128 (little endian in x0, x1) -> the eight
// exact fp16 values b: 0x6400 | u is the half 1024 + u
__device__ __forceinline__ h8 u8x8_to_h8(uint32_t x0, uint32_t x1) {
    const h2 bias = {(_Float16)-1152.f, (_Float16)-1152.f};
    const h2 a = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, x0, 0x04010400u)) + bias;
    const h2 b = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, x0, 0x04030402u)) + bias;
    const h2 c = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, x1, 0x04010400u)) + bias;
    const h2 d = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, x1, 0x04030402u)) + bias;
    const h8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    return r;
}

// Encode one token (quantise K; sign flip, fast Walsh-Hadamard transform,
// quantise V) and write it at cache row prow (kv-head base + position): one
// wave, lane holding dims P lane .. P lane + P - 1; vq is D bytes of LDS.
template <int D, int FMT = 0>
__device__ void encode_append(const float* kp, const float* vp, const float* signs, int8_t* kc, uint16_t* ks,
                              uint32_t* vc, uint16_t* vs, int64_t prow, uint8_t* vq, int lane,
                              _Float16* kwr = nullptr, _Float16* vwr = nullptr) {
    typedef KvFmt<FMT> F;
    constexpr int NG = D / 32, NB = D / 16, VW = F::FB * D / 32;
    const float qscale = 1.0f / sqrtf((float)D);
    constexpr int P = D / 64;                 // dims per lane: d = P lane + i
    constexpr int GL = 32 / P;                // lanes per scale group
    float kv[P], v[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        kv[i] = kp[P * lane + i];
        v[i] = F::ROT ? vp[P * lane + i] * signs[P * lane + i] : vp[P * lane + i];
    }
    // recent window (kwr non-null): the fp32 key and, below, the fp32 rotated
    // value are also kept rounded to fp16
    if (kwr)
#pragma unroll
        for (int i = 0; i < P; ++i) kwr[P * lane + i] = (_Float16)kv[i];
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < P; ++i) am = fmaxf(am, fabsf(kv[i]));
#pragma unroll
    for (int o = 1; o < GL; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
    if (F::KB == 8) {
        const _Float16 sh = (_Float16)(am / 127.0f);
        const float sc = (float)sh;
        uint32_t packed = 0;
#pragma unroll
        for (int i = 0; i < P; ++i) {
            float cd = sc == 0.f ? 0.f : rintf(kv[i] / sc);
            cd = fminf(fmaxf(cd, -127.f), 127.f);
            packed |= (uint32_t)((int)cd + 128) << (8 * i);
        }
        // P consecutive dims stay consecutive bytes of the permuted row
        if (P == 4) *(uint32_t*)(kc + prow * D + k_byte<D>(P * lane)) = packed;
        else kc[prow * D + k_byte<D>(lane)] = (int8_t)(uint8_t)packed;
        if (lane % GL == 0) ks[prow * NG + lane / GL] = __builtin_bit_cast(uint16_t, sh);
    } else {
        // 4-bit keys: dim 32 g + 8 q + e goes to nibble slot [0,2,4,6,1,3,5,7][e]
        // of dword q NG + g; the 8 / P lanes sharing a dword merge their nibbles
        const _Float16 sh = (_Float16)(am / 7.0f);
        const float sc = (float)sh;
        uint32_t part = 0;
#pragma unroll
        for (int i = 0; i < P; ++i) {
            float cd = sc == 0.f ? 0.f : rintf(kv[i] / sc);
            cd = fminf(fmaxf(cd, -7.f), 7.f);
            const int d = P * lane + i, e = d & 7;
            part |= (uint32_t)((int)cd + 8) << (4 * w4_slot(e));
        }
#pragma unroll
        for (int o = 1; o < 8 / P; o <<= 1) part |= __shfl_xor(part, o, 64);
        const int d0 = P * lane;
        if ((d0 & 7) == 0) {
            const int g = d0 >> 5, qq = (d0 & 31) >> 3;
            ((uint32_t*)kc)[prow * (D / 8) + qq * NG + g] = part;
        }
        if (lane % GL == 0) ks[prow * NG + lane / GL] = __builtin_bit_cast(uint16_t, sh);
    }
    // Sylvester transform, stage by stage in the order of the index bits
#pragma unroll
    for (int hh = 1; hh < D && F::ROT; hh <<= 1) {
        if (hh < P) {
#pragma unroll
            for (int i = 0; i < P; ++i)
                if ((i & hh) == 0) {
                    const float x = v[i], y = v[i + hh];
                    v[i] = x + y;
                    v[i + hh] = x - y;
                }
        } else {
            const int lm = hh / P;
#pragma unroll
            for (int i = 0; i < P; ++i) {
                const float o = __shfl_xor(v[i], lm, 64);
                v[i] = (lane & lm) ? o - v[i] : v[i] + o;
            }
        }
    }
    am = 0.f;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        if (F::ROT) v[i] *= qscale;   // 1/sqrt(D): a power of two for D = 64, 256
        am = fmaxf(am, fabsf(v[i]));
        ss += v[i] * v[i];
    }
    if (vwr)
#pragma unroll
        for (int i = 0; i < P; ++i) vwr[P * lane + i] = (_Float16)v[i];
#pragma unroll
    for (int o = 1; o < GL; o <<= 1) {
        am = fmaxf(am, __shfl_xor(am, o, 64));
        ss += __shfl_xor(ss, o, 64);
    }
    if (FMT == 2) {
        // codebook: scale fp16(root mean square), the nearest level of v / s
        // (ties to the lower level) as a sign-magnitude field
        const _Float16 sh = (_Float16)sqrtf(ss / 32.0f);
        const float sc = (float)sh;
        const float l0 = (float)(_Float16)0.2451f, l1 = (float)(_Float16)0.7560f, l2 = (float)(_Float16)1.3440f,
                    l3 = (float)(_Float16)2.1520f;
        const float m01 = 0.5f * (l0 + l1), m12 = 0.5f * (l1 + l2), m23 = 0.5f * (l2 + l3);
#pragma unroll
        for (int i = 0; i < P; ++i) {
            int f = 0;   // sc == 0: level +0.2451 x 0
            if (sc != 0.f) {
                const float t = v[i] / sc;
                const int c = (t > -m23) + (t > -m12) + (t > -m01) + (t > 0.f) + (t > m01) + (t > m12) + (t > m23);
                f = c >= 4 ? c - 4 : 7 - c;
            }
            vq[P * lane + i] = (uint8_t)f;
        }
        if (lane % GL == 0) vs[prow * NG + lane / GL] = __builtin_bit_cast(uint16_t, sh);
    } else {
        constexpr float vq_max = FMT == 1 ? 7.0f : 3.0f;
        constexpr int vq_off = FMT == 1 ? 8 : 4;
        const _Float16 sh = (_Float16)(am / vq_max);
        const float sc = (float)sh;
#pragma unroll
        for (int i = 0; i < P; ++i) {
            float cd = sc == 0.f ? 0.f : rintf(v[i] / sc);
            cd = fminf(fmaxf(cd, -vq_max), vq_max);
            vq[P * lane + i] = (uint8_t)((int)cd + vq_off);
        }
        if (lane % GL == 0) vs[prow * NG + lane / GL] = __builtin_bit_cast(uint16_t, sh);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < VW) {
        // word lane of the record: FB-bit fields f = NB (d % 16) + d / 16 overlapping its bits
        uint32_t word = 0;
        const int lo = 32 * lane;
        const int f0 = lo / F::FB > 0 ? lo / F::FB - 1 : 0;
        const int f1 = min(D - 1, (lo + 31) / F::FB);
        for (int f = f0; f <= f1; ++f) {
            const int d = 16 * (f % NB) + f / NB;
            const uint32_t n = vq[d];
            const int sft = F::FB * f - lo;
            if (sft >= 32 || sft <= -F::FB) continue;
            word |= sft >= 0 ? n << sft : n >> (-sft);
        }
        vc[prow * VW + lane] = word;
    }
    __threadfence_block();
}

// NT tokens at consecutive positions share one sweep over the cache: query
// column c of the score product is token c / G, head c % G (QC = G NT <= 16
// columns), and token m sees positions up to its own.  Grid z: blocks of NT
// tokens of a longer run (a prefill chunk), block b taking tokens b NT ...
template <int D, int G, int NT, int FMT = 0>
__global__ __launch_bounds__(512, 1) void k_attn(AttnArgs a) {
    typedef KvFmt<FMT> F;
    constexpr int NG = D / 32;          // scale groups
    constexpr int NB = D / 16;          // 16-dim blocks of the value product
    constexpr int VW = F::FB * NG;      // 32-bit words per value record
    constexpr int VB = F::FB * NB;      // value bits per lane slot
    constexpr int KROW = D * F::KB / 8; // key bytes per position
    constexpr int KW = NG * F::KB / 4;  // key dwords a lane loads per position (its quarter)
    constexpr int HPL = NG / 2;         // staged scale halves per lane (NG >= 2)
    constexpr int QC = G * NT;          // query columns
    static_assert(G >= 1 && QC <= 16 && NG >= 2, "shape");
    // wave results merge in one pass when all fit 48 KB, else through 4 slots
    constexpr bool kOnePass = kWaves * QC * D <= 12288;

    __shared__ uint8_t vq[D];
    __shared__ float stile[kWaves][2][NG][kTile];      // per wave: key / value scales [group][position]
    __shared__ float mo[kOnePass ? kWaves : 4][QC][D];  // wave results
    __shared__ float mm[kWaves][QC], ll[kWaves][QC];

    const int j = blockIdx.y, tid = threadIdx.x;
    // split and token block: grid (split, kv head, block), or with zfast the
    // nz token blocks of a split next to each other in x, and with two blocks
    // and whole groups of 8 splits eight apart, so that both run at the same
    // time on one XCD (workgroups are dealt to the 8 XCDs in turn) and the
    // later block's cache reads find the earlier one's lines in its L2
    int split = blockIdx.x, zb = blockIdx.z;
    if (NT > 1 && a.zfast) {
        const int nz = (a.nt + NT - 1) / NT, b = blockIdx.x;
        if (nz == 2 && a.nsplit % 8 == 0) {
            zb = (b >> 3) & 1;
            split = ((b >> 4) << 3) | (b & 7);
        } else {
            zb = b % nz;
            split = b / nz;
        }
    }
    const int tb0 = zb * NT;                  // the block's first token in the run
    const int lane = tid & 63, w = tid >> 6;
    const int c = lane & 15, q = lane >> 4;
    // the block's first token's position; in a batch each block is a sequence
    // with its own cache
    const int pos = a.batch ? a.pos[blockIdx.z] : *a.pos + a.pos_offset + tb0;
    const int64_t zoff = a.batch ? (int64_t)blockIdx.z * a.seq_bytes : 0;
    int8_t* const kc = (int8_t*)((char*)a.kc + zoff);
    uint16_t* const ks = (uint16_t*)((char*)a.ks + zoff);
    uint32_t* const vc = (uint32_t*)((char*)a.vc + zoff);
    uint16_t* const vs = (uint16_t*)((char*)a.vs + zoff);
    const int nt = NT == 1 ? 1 : min(NT, a.nt - tb0);
    // with a recent window (win > 0) this sweep covers only the positions
    // before it; k_attn_win reads the window.  With zfast one combine merges
    // every token of the run, so every block splits the positions up to the
    // run's end (the combine's partition) and masks those after its tokens.
    const int npos = (NT > 1 && a.zfast ? *a.pos + a.pos_offset + a.nt : pos + nt) - (a.win > 0 ? a.win : 0);
    if (npos <= 0) return;
    int pps, used;
    split_range(npos, a.nsplit, pps, used);
    if (split >= used) return;
    const int t0 = split * pps;
    const int t1 = min(npos, t0 + pps);
    const int64_t hbase = (int64_t)j * a.max_ctx;
    const float qscale = 1.0f / sqrtf((float)D);

    // raw words of one tile for this lane
    struct Raw {
        uint32_t k[KW];            // key codes of position tile0 + c, quarter q
        uint32_t vlo[4], vhi[4];   // value words of positions tile0 + 4 q + r
        uint32_t sc[2];            // HPL staged scale halves
        bool sv;                   // their position is inside the range
    };
    const int vbit0 = VB * c;
    const int vw0 = vbit0 >> 5, vsh = vbit0 & 31;
    const int vw1 = vw0 + 1 < VW ? vw0 + 1 : VW - 1;
    // scale staging: lanes 0..31 key scales, 32..63 value scales; HPL halves each
    const int ssel = lane >> 5;
    const int sidx = (lane & 31) * HPL;
    const int spp = sidx / NG, sg0 = sidx % NG;
    const uint16_t* sbase = ssel ? vs : ks;

    // per-head bases; offsets inside a head fit 32 bits (max_ctx * D < 2^31)
    const int8_t* khead = kc + hbase * KROW;
    const uint32_t* vhead = vc + hbase * VW;
    const uint16_t* shead = sbase + hbase * NG;
    auto load = [&](int tile0, Raw& r) {
        {
            const int p = min(tile0 + c, t1 - 1);
            const uint32_t* kp = (const uint32_t*)(khead + (p * KROW + 4 * KW * q));
            if (KW % 4 == 0) {
#pragma unroll
                for (int i = 0; i < KW / 4; ++i) {
                    const uint4 x = ((const uint4*)kp)[i];
                    r.k[4 * i] = x.x; r.k[4 * i + 1] = x.y; r.k[4 * i + 2] = x.z; r.k[4 * i + 3] = x.w;
                }
            } else {
#pragma unroll
                for (int i = 0; i < KW / 2; ++i) {
                    const uint2 x = ((const uint2*)kp)[i];
                    r.k[2 * i] = x.x; r.k[2 * i + 1] = x.y;
                }
            }
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const uint32_t* rec = vhead + min(tile0 + 4 * q + rr, t1 - 1) * VW;
            r.vlo[rr] = rec[vw0];
            r.vhi[rr] = rec[vw1];
        }
        {
            const int p = tile0 + spp;
            const uint16_t* sp = shead + (min(p, t1 - 1) * NG + sg0);
            if (HPL == 4) {
                const uint2 v = *(const uint2*)sp;
                r.sc[0] = v.x;
                r.sc[1] = v.y;
            } else if (HPL == 2) {
                r.sc[0] = *(const uint32_t*)sp;
                r.sc[1] = 0u;
            } else {
                r.sc[0] = *sp;
                r.sc[1] = 0u;
            }
            r.sv = p < t1;
        }
    };

    // The current token is encoded (quantise K; sign flip, fast Walsh-Hadamard
    // transform, quantise V) and appended by one wave: the one that owns the
    // final tile of the range that ends at it.  Only that tile holds the new
    // position, so no other wave waits; the writer's own loads of that tile
    // come after its stores in program order.
    auto encode = [&]() {
        const float* kp = a.proj + (int64_t)tb0 * a.sproj + 2LL * a.nq * D + (int64_t)j * D;
        encode_append<D, FMT>(kp, kp + (int64_t)a.nkv * D, a.signs, kc, ks, vc, vs, hbase + pos, vq, lane);
    };

    const int ntiles = (t1 - t0 + kTile - 1) / kTile;
    const bool writer = NT == 1 && a.append && t1 == npos && w == (ntiles - 1) % kWaves;
    const bool first_final = w == ntiles - 1;
    Raw cur = {}, nxt = {};
    // the first tile is in flight while q is read; the writer requests the
    // final tile only after appending the token
    if (w < ntiles && !(writer && first_final)) load(t0 + w * kTile, cur);
    if (writer) {
        encode();
        if (first_final) load(t0 + w * kTile, cur);
    }

    // query fragments (B operand of the score product): head c, dims 32 g + 8 q + e,
    // pre-scaled by 1/sqrt(D), as fp16 hi + lo so the scores keep fp32 accuracy
    const bool qv = c < G * nt;                        // a live query column
    const int cm = qv ? c / G : 0, cg = qv ? c % G : 0;
    const int lim = pos + cm;                          // last position column c sees
    h8 qh[NG], ql[NG];
    {
        // every lane loads (a dead column reads column 0) and all loads are
        // pinned before the first use: guarded loads were sunk into one branch
        // and one full memory wait per group
        const float* qp = a.proj + (int64_t)(tb0 + cm) * a.sproj + (int64_t)(j * G + cg) * D + 8 * q;
        f4 xq[NG][2];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            xq[g][0] = *(const f4*)(qp + 32 * g);
            xq[g][1] = *(const f4*)(qp + 32 * g + 4);
        }
#pragma unroll
        for (int g = 0; g < NG; ++g) asm volatile("" : "+v"(xq[g][0]), "+v"(xq[g][1]));
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float xs[8] = {xq[g][0][0], xq[g][0][1], xq[g][0][2], xq[g][0][3],
                                 xq[g][1][0], xq[g][1][1], xq[g][1][2], xq[g][1][3]};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = qv ? xs[e] * qscale : 0.f;
                const _Float16 hi = (_Float16)v;
                qh[g][e] = hi;
                ql[g][e] = (_Float16)(v - (float)hi);
            }
        }
    }

    float m = -INFINITY, l = 0.f;
    f4 o[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) o[b] = f4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int tile0, const Raw& r) {
        // stage this tile's scales, transposed to [group][position]; positions
        // past the range get zero scales
#pragma unroll
        for (int h = 0; h < HPL; ++h)
            stile[w][ssel][sg0 + h][spp] =
                r.sv ? (float)__builtin_bit_cast(_Float16, (uint16_t)(r.sc[h >> 1] >> (16 * (h & 1)))) : 0.f;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // scores of head c at positions tile0 + 4 q + rr
        float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const h8 kf = F::KB == 4 ? nib8_to_h8(r.k[g]) : u8x8_to_h8(r.k[2 * g], r.k[2 * g + 1]);
            f4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qh[g], (f4{0.f, 0.f, 0.f, 0.f}), 0, 0, 0);
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, ql[g], d, 0, 0, 0);
            const f4 ks = *(const f4*)&stile[w][0][g][4 * q];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) s[rr] += ks[rr] * d[rr];
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            if (tile0 + 4 * q + rr >= t1 || (NT > 1 && tile0 + 4 * q + rr > lim)) s[rr] = -INFINITY;

        // online softmax for column c (the four quarters hold the tile's 16
        // positions); with several tokens a column can see none of a tile
        float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mn = fmaxf(m, mx);
        const bool none = NT > 1 && mn == -INFINITY;
        const float corr = none ? 1.f : __expf(m - mn);
        float p[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) p[rr] = none ? 0.f : __expf(s[rr] - mn);
        l = l * corr + ((p[0] + p[1]) + (p[2] + p[3]));
        m = mn;
        if (__builtin_amdgcn_ballot_w64(corr != 1.0f)) {
#pragma unroll
            for (int b = 0; b < NB; ++b) o[b] *= corr;
        }

        // O^T += V^T P'^T, 16 dims per MFMA, with P' = p x value scale of the
        // position's group in fp32, split into fp16 hi + lo (round toward zero;
        // the lo part carries the residual) so that the product keeps fp32
        // accuracy; the codes themselves are exact halves.  The lane's value slot
        // of position rr holds dims c + 16 b at bits 3 b.
        uint32_t lo32[4], mid[4], hi32[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const uint64_t win = ((((uint64_t)r.vhi[rr]) << 32) | r.vlo[rr]) >> vsh;
            lo32[rr] = (uint32_t)win;
            mid[rr] = (uint32_t)(win >> 16);
            hi32[rr] = (uint32_t)(win >> 32);
        }
        // 3-bit fields of positions (0, 1) and (2, 3) five at a time: the low
        // 16 bits of each position's shifted slot side by side in one word;
        // 4-bit fields four at a time, from each 16-bit quarter of the slot
        uint32_t zc[2][4];
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
            const int ra = 2 * pr, rb = 2 * pr + 1;
            if (F::FB == 4) {
                zc[pr][0] = __builtin_amdgcn_perm(lo32[rb], lo32[ra], 0x05040100u);                 // fields 0..3
                if (NB > 4) zc[pr][1] = __builtin_amdgcn_perm(lo32[rb], lo32[ra], 0x07060302u);     // 4..7
                if (NB > 8) zc[pr][2] = __builtin_amdgcn_perm(hi32[rb], hi32[ra], 0x05040100u);     // 8..11
                if (NB > 12) zc[pr][3] = __builtin_amdgcn_perm(hi32[rb], hi32[ra], 0x07060302u);    // 12..15
            } else {
                zc[pr][0] = __builtin_amdgcn_perm(lo32[rb], lo32[ra], 0x05040100u);               // fields 0..4
                if (NB > 5) zc[pr][1] = __builtin_amdgcn_perm(lo32[rb] >> 15, lo32[ra] >> 15, 0x05040100u);  // 5..9
                if (NB > 10) zc[pr][2] = __builtin_amdgcn_perm(mid[rb] >> 14, mid[ra] >> 14, 0x05040100u);  // 10..14
                if (NB > 15) zc[pr][3] = __builtin_amdgcn_perm(mid[rb] >> 29, mid[ra] >> 29, 0x05040100u);  // 15
            }
        }
        uint32_t lmt_lo = 0, lmt_hi = 0;
        if (FMT == 2) lm_table(lmt_lo, lmt_hi);
        const h2 bias = {(_Float16)-1028.f, (_Float16)-1028.f};
        const h2 bias4 = {(_Float16)-1032.f, (_Float16)-1032.f};
        // (x & mask) | 0x6400 halves in one v_and_or_b32: the mask in an SGPR and
        // the constant in a VGPR (a gfx9 VOP3 takes no literal operands)
        uint32_t m7, h64;
        asm volatile("s_mov_b32 %0, 0x70007" : "=s"(m7));
        asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(h64));
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const f4 vs = *(const f4*)&stile[w][1][g][4 * q];
            float pg[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) pg[rr] = p[rr] * vs[rr];
            const h2 hi01 = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(pg[0], pg[1]));
            const h2 hi23 = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(pg[2], pg[3]));
            const h2 lo01 = __builtin_bit_cast(
                h2, __builtin_amdgcn_cvt_pkrtz(pg[0] - (float)hi01[0], pg[1] - (float)hi01[1]));
            const h2 lo23 = __builtin_bit_cast(
                h2, __builtin_amdgcn_cvt_pkrtz(pg[2] - (float)hi23[0], pg[3] - (float)hi23[1]));
            const h4 phi = {hi01[0], hi01[1], hi23[0], hi23[1]};
            const h4 plo = {lo01[0], lo01[1], lo23[0], lo23[1]};
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const int b = 2 * g + bb;
                h2 v01, v23;
                if (F::FB == 4) {
                    const int ch = b / 4, sh4 = 4 * (b % 4);
                    v01 = __builtin_bit_cast(h2, ((zc[0][ch] >> sh4) & 0x000F000Fu) | 0x64006400u) + bias4;
                    v23 = __builtin_bit_cast(h2, ((zc[1][ch] >> sh4) & 0x000F000Fu) | 0x64006400u) + bias4;
                } else if (FMT == 2) {
                    const int ch = b / 5, sh3 = 3 * (b % 5);
                    v01 = lm_pair(zc[0][ch] >> sh3, lmt_lo, lmt_hi);
                    v23 = lm_pair(zc[1][ch] >> sh3, lmt_lo, lmt_hi);
                } else {
                    const int ch = b / 5, sh3 = 3 * (b % 5);
                    v01 = __builtin_bit_cast(h2, ((zc[0][ch] >> sh3) & m7) | h64) + bias;
                    v23 = __builtin_bit_cast(h2, ((zc[1][ch] >> sh3) & m7) | h64) + bias;
                }
                const h4 va = {v01[0], v01[1], v23[0], v23[1]};
                o[b] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, phi, o[b], 0, 0, 0);
                o[b] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, plo, o[b], 0, 0, 0);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
    };

    {
        // the next tile's loads are issued before the current tile is used; the
        // last round re-reads the final tile so every round issues the same loads
        // two register sets used in turn (no copies between rounds)
        for (int tt = w; tt < ntiles; tt += 2 * kWaves) {
            load(t0 + min(tt + kWaves, ntiles - 1) * kTile, nxt);
            compute(t0 + tt * kTile, cur);
            if (tt + kWaves >= ntiles) break;
            load(t0 + min(tt + 2 * kWaves, ntiles - 1) * kTile, cur);
            compute(t0 + (tt + kWaves) * kTile, nxt);
        }
    }
    // the four quarters hold partial sums of l for head c
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);

    // partial rows: column c of kv head j is slot (c / G) nq + j G + c % G
    // partial rows hold nsplit + nsplit_w split slots (the window's last)
    const int sstride = a.nsplit + a.nsplit_w;
    float* mlp = a.part + (int64_t)a.prow * sstride * D;
    auto slot_row = [&](int cc) { return (int64_t)((tb0 + cc / G) * a.nq + j * G + cc % G) * sstride + split; };
    if (kOnePass) {
        // every wave posts (m, l, acc) of its columns; lane (c, q) holds column c,
        // dims 16 b + 4 q + rr; then one pass merges the waves per output
        if (c < QC) {
#pragma unroll
            for (int b = 0; b < NB; ++b) *(f4*)&mo[w][c][16 * b + 4 * q] = o[b];
            if (q == 0) {
                mm[w][c] = m;
                ll[w][c] = l;
            }
        }
        __syncthreads();
        for (int idx = tid; idx < G * nt * D; idx += 64 * kWaves) {
            const int g = idx / D, e = idx % D;
            float M = mm[0][g];
#pragma unroll
            for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, mm[ww][g]);
            float L = 0.f, A = 0.f;
#pragma unroll
            for (int ww = 0; ww < kWaves; ++ww) {
                const float f = mm[ww][g] == -INFINITY ? 0.f : __expf(mm[ww][g] - M);
                L += ll[ww][g] * f;
                A += mo[ww][g][e] * f;
            }
            const int64_t row = slot_row(g);
            a.part[row * D + e] = A;
            if (e == 0) {
                mlp[2 * row] = M;
                mlp[2 * row + 1] = L;
            }
        }
    } else {
        // the waves first agree on each column's maximum and rescale to it,
        // then add their accumulators through four LDS slots
        if (c < QC && q == 0) {
            mm[w][c] = m;
            ll[w][c] = l;
        }
        __syncthreads();
        {
            float M = -INFINITY;
            if (c < QC)
#pragma unroll
                for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, mm[ww][c]);
            const float f = m == -INFINITY ? 0.f : __expf(m - M);
#pragma unroll
            for (int b = 0; b < NB; ++b) o[b] *= f;
        }
        if (w >= 4 && c < QC)
#pragma unroll
            for (int b = 0; b < NB; ++b) *(f4*)&mo[w - 4][c][16 * b + 4 * q] = o[b];
        __syncthreads();
        if (w < 4 && c < QC)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                f4* slot = (f4*)&mo[w][c][16 * b + 4 * q];
                *slot = o[b] + *slot;
            }
        __syncthreads();
        for (int idx = tid; idx < G * nt * D; idx += 64 * kWaves) {
            const int g = idx / D, e = idx % D;
            float M = mm[0][g];
#pragma unroll
            for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, mm[ww][g]);
            float L = 0.f;
#pragma unroll
            for (int ww = 0; ww < kWaves; ++ww) L += ll[ww][g] * (mm[ww][g] == -INFINITY ? 0.f : __expf(mm[ww][g] - M));
            const float A = (mo[0][g][e] + mo[1][g][e]) + (mo[2][g][e] + mo[3][g][e]);
            const int64_t row = slot_row(g);
            a.part[row * D + e] = A;
            if (e == 0) {
                mlp[2 * row] = M;
                mlp[2 * row + 1] = L;
            }
        }
    }
}

// KMAX: split rows per thread, enough for the launch's split count; ROT: the
// values were cached in the rotated domain, so the merged row is rotated back
template <int D, int KMAX, bool ROT = true>
__global__ __launch_bounds__(1024) void k_combine(CombineArgs a) {
    constexpr int LR = D / 4;            // lanes per split row, a float4 each
    constexpr int ROWS = 1024 / LR;      // split rows in flight
    constexpr int P = D / 64;            // values per lane in the final transform
    __shared__ float wts[256];
    __shared__ float red[ROWS][D];
    __shared__ float v[D];
    __shared__ float rmax[16], rsum[16];
    // block i: token i / nq, head i % nq (its slot in the partial rows)
    const int i = blockIdx.x, tid = threadIdx.x;
    const int tm = i / a.nq, hq = i % a.nq;
    int pps, used;
    const int npos_all = a.batch ? a.pos[tm] + 1 : *a.pos + a.pos_offset + a.nt;
    // with a recent window: splits of the positions before it (slots 0 ..
    // used_q - 1), then the window's splits (slots nsplit ..)
    const int nq_pos = npos_all - (a.win > 0 ? a.win : 0);
    int used_q = 0;
    if (nq_pos > 0) split_range(nq_pos, a.nsplit, pps, used_q);
    int used_w = 0;
    if (a.win > 0) split_range(npos_all < a.win ? npos_all : a.win, a.nsplit_w, pps, used_w);
    used = used_q + used_w;
    const int sstride = a.nsplit + a.nsplit_w;
    auto slot = [&](int sp) { return sp < used_q ? sp : a.nsplit + (sp - used_q); };
    const float* base = a.part + (int64_t)i * sstride * D;
    const float* mlp = a.part + (int64_t)a.prow * sstride * D + 2LL * i * sstride;
    // every load is issued before any is used: (m, l) of one split per
    // thread, then this thread's slices of the split rows
    float ms = -INFINITY, ls = 0.f;
    if (tid < used) {
        ms = mlp[2 * slot(tid)];
        ls = mlp[2 * slot(tid) + 1];
    }
    // the output gate of this head, for the wave that finishes (lane holds
    // dims P lane .. P lane + P - 1), requested with the rest
    float gate[P], sgn[P];
    {
        const float* gp = a.proj + (int64_t)tm * a.sproj + (int64_t)a.nq * D + (int64_t)hq * D + P * (tid & 63);
#pragma unroll
        for (int j = 0; j < P; ++j) {
            gate[j] = gp[j];
            sgn[j] = a.signs[P * (tid & 63) + j];
        }
    }
    // straight-line loads (a split past `used` re-reads split 0 and is
    // dropped), pinned before the first use so that none is sunk into a
    // branch with a wait of its own; KMAX fits the launch's split count, so
    // few of them are dead
    const int row = tid / LR, e4 = tid % LR;
    f4 pv[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const int sp = row + k * ROWS;
        pv[k] = *(const f4*)(base + (int64_t)(sp < used ? slot(sp) : 0) * D + 4 * e4);
    }
#pragma unroll
    for (int k = 0; k < KMAX; ++k) asm volatile("" : "+v"(pv[k]));
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        if (row + k * ROWS >= used) pv[k] = f4{0.f, 0.f, 0.f, 0.f};
    // split weights exp(m_s - M) and the normaliser
    float M = ms;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    if ((tid & 63) == 0) rmax[tid >> 6] = M;
    __syncthreads();
    M = rmax[0];
#pragma unroll
    for (int k = 1; k < 16; ++k) M = fmaxf(M, rmax[k]);
    const float wgt = tid < used ? __expf(ms - M) : 0.f;
    if (tid < 256) wts[tid] = wgt;
    float L = wgt * ls;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o, 64);
    if ((tid & 63) == 0) rsum[tid >> 6] = L;
    __syncthreads();
    L = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) L += rsum[k];
    {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int sp = row + k * ROWS;
            if (sp < used) acc += wts[sp] * pv[k];
        }
        *(f4*)&red[row][4 * e4] = acc;
    }
    __syncthreads();
    if (tid < D) {
        float t = 0.f;
#pragma unroll
        for (int r = 0; r < ROWS; ++r) t += red[r][tid];
        v[tid] = t / L;
    }
    __syncthreads();
    if (!ROT && tid < 64) {
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const int d = P * tid + j;
            a.out[(int64_t)i * D + d] = (_Float16)(v[d] * sigmoidf_(gate[j]));
        }
    }
    if (ROT && tid < 64) {
        // undo the rotation in one wave: Sylvester transform stage by stage in
        // the order of the index bits, lane holds d = P lane + j
        const int lane = tid;
        float x[P];
#pragma unroll
        for (int j = 0; j < P; ++j) x[j] = v[P * lane + j];
#pragma unroll
        for (int hh = 1; hh < D; hh <<= 1) {
            if (hh < P) {
#pragma unroll
                for (int j = 0; j < P; ++j)
                    if ((j & hh) == 0) {
                        const float p0 = x[j], p1 = x[j + hh];
                        x[j] = p0 + p1;
                        x[j + hh] = p0 - p1;
                    }
            } else {
                const int lm = hh / P;
#pragma unroll
                for (int j = 0; j < P; ++j) {
                    const float o = __shfl_xor(x[j], lm, 64);
                    x[j] = (lane & lm) ? o - x[j] : x[j] + o;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const int d = P * lane + j;
            const float o = x[j] * (1.0f / sqrtf((float)D)) * sgn[j];
            a.out[(int64_t)i * D + d] = (_Float16)(o * sigmoidf_(gate[j]));
        }
    }
}

// The nt tokens' K and V at positions *pos + pos_offset + m, one wave per
// (kv head, token), before a multi-token sweep reads them.
template <int D>
__global__ __launch_bounds__(64) void k_append(AttnArgs a) {
    __shared__ uint8_t vq[D];
    const int j = blockIdx.x, tm = blockIdx.y;
    const int pos = *a.pos + a.pos_offset + tm;
    const float* kp = a.proj + (int64_t)tm * a.sproj + 2LL * a.nq * D + (int64_t)j * D;
    _Float16 *kwr = nullptr, *vwr = nullptr;
    if (a.win > 0) {
        const int64_t wr = ((int64_t)j * a.win + pos % a.win) * D;
        kwr = a.kw + wr;
        vwr = a.vw + wr;
    }
    encode_append<D>(kp, kp + (int64_t)a.nkv * D, a.signs, a.kc, a.ks, a.vc, a.vs, (int64_t)j * a.max_ctx + pos, vq,
                     threadIdx.x, kwr, vwr);
}

// The recent window of the single-token decode step: positions
// [npos - win, npos) of kv head blockIdx.y, read at fp16 from the ring
// (position t at slot t % win, [nkv][win][D]), split over gridDim.x
// workgroups whose partial rows go to slots nsplit + split, in the layout the
// quantised sweep uses, so that k_combine merges both.  Lane l holds dims
// P l .. P l + P - 1 of the G query heads and of each position's key and value
// (a wave's row load is one contiguous 2 D-byte run).  Rounds of
// kWinWaves x kWinPer positions: each wave requests all of its kWinPer rows
// before using any, reduces the scores across the wave with DPP moves and
// keeps an online softmax per head; the waves merge through LDS.
constexpr int kWinWaves = 8;
constexpr int kWinPer = 8;

__device__ __forceinline__ float wave_sum_dpp(float v) {
#define AW4_WDPP(ctrl)                                                                                   \
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, 0xF, \
                                                               0xF, true))
    AW4_WDPP(0xB1);    // quad_perm [1,0,3,2]
    AW4_WDPP(0x4E);    // quad_perm [2,3,0,1]
    AW4_WDPP(0x141);   // row_half_mirror
    AW4_WDPP(0x140);   // row_mirror
#undef AW4_WDPP
    const int iv = __builtin_bit_cast(int, v);
    return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 0)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 16))) +
           (__builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 32)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 48)));
}

template <int D, int G>
__global__ __launch_bounds__(64 * kWinWaves) void k_attn_win(AttnArgs a) {
    constexpr int P = D / 64;
    typedef _Float16 hP __attribute__((ext_vector_type(P)));
    __shared__ float mo[kWinWaves][G][D];
    __shared__ float mm[kWinWaves][G], ll[kWinWaves][G];
    __shared__ uint8_t vq[D];
    const int split = blockIdx.x, j = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int npos = *a.pos + a.pos_offset + 1;
    const int wlen = npos < a.win ? npos : a.win;
    int pps, used;
    split_range(wlen, a.nsplit_w, pps, used);
    if (split >= used) return;
    const int t0 = npos - wlen + split * pps;
    const int t1 = min(npos, t0 + pps);
    // append (a.append): the wave that owns the token's position encodes it
    // (codes and ring entry) before it reads its rows; no other wave or
    // workgroup reads that position
    if (a.append && t1 == npos && w == (npos - 1 - t0) % kWinWaves) {
        const float* kp = a.proj + 2LL * a.nq * D + (int64_t)j * D;
        const int64_t wr = ((int64_t)j * a.win + (npos - 1) % a.win) * D;
        encode_append<D>(kp, kp + (int64_t)a.nkv * D, a.signs, a.kc, a.ks, a.vc, a.vs,
                         (int64_t)j * a.max_ctx + npos - 1, vq, lane, a.kw + wr, a.vw + wr);
    }
    const float qscale = 1.0f / sqrtf((float)D);
    const hP* kb = (const hP*)(a.kw + (int64_t)j * a.win * D) + lane;
    const hP* vb = (const hP*)(a.vw + (int64_t)j * a.win * D) + lane;
    float q[G][P];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < P; ++i) q[h][i] = a.proj[(int64_t)(j * G + h) * D + P * lane + i] * qscale;
    float m[G], l[G], acc[G][P];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int i = 0; i < P; ++i) acc[h][i] = 0.f;
    }
    for (int base = t0 + w; base < t1; base += kWinWaves * kWinPer) {
        // this round's rows, all requested first (a position past the split
        // re-reads the first one and gets no weight)
        hP kr[kWinPer], vr[kWinPer];
#pragma unroll
        for (int r = 0; r < kWinPer; ++r) {
            const int t = base + kWinWaves * r;
            const int64_t row = (int64_t)((t < t1 ? t : base) % a.win) * (D / P);
            kr[r] = kb[row];
            vr[r] = vb[row];
        }
        // every score of the round first (independent wave reductions), then
        // one online-softmax update per head
        float sc[kWinPer][G];
#pragma unroll
        for (int r = 0; r < kWinPer; ++r)
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float sdot = 0.f;
#pragma unroll
                for (int i = 0; i < P; ++i) sdot += q[h][i] * (float)kr[r][i];
                sc[r][h] = base + kWinWaves * r < t1 ? wave_sum_dpp(sdot) : -INFINITY;
            }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mn = m[h];
#pragma unroll
            for (int r = 0; r < kWinPer; ++r) mn = fmaxf(mn, sc[r][h]);
            const float corr = __expf(m[h] - mn);   // 0 while m = -inf
            l[h] *= corr;
#pragma unroll
            for (int i = 0; i < P; ++i) acc[h][i] *= corr;
#pragma unroll
            for (int r = 0; r < kWinPer; ++r) {
                const float pe = __expf(sc[r][h] - mn);   // 0 for a dead position
                l[h] += pe;
#pragma unroll
                for (int i = 0; i < P; ++i) acc[h][i] += pe * (float)vr[r][i];
            }
            m[h] = mn;
        }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int i = 0; i < P; ++i) mo[w][h][P * lane + i] = acc[h][i];
        if (lane == 0) {
            mm[w][h] = m[h];
            ll[w][h] = l[h];
        }
    }
    __syncthreads();
    const int sstride = a.nsplit + a.nsplit_w;
    float* mlp = a.part + (int64_t)a.prow * sstride * D;
    for (int idx = tid; idx < G * D; idx += 64 * kWinWaves) {
        const int h = idx / D, e = idx % D;
        float M = mm[0][h];
#pragma unroll
        for (int ww = 1; ww < kWinWaves; ++ww) M = fmaxf(M, mm[ww][h]);
        float L = 0.f, A = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWinWaves; ++ww) {
            const float f = mm[ww][h] == -INFINITY ? 0.f : __expf(mm[ww][h] - M);
            L += ll[ww][h] * f;
            A += mo[ww][h][e] * f;
        }
        const int64_t row = (int64_t)(j * G + h) * sstride + a.nsplit + split;
        a.part[row * D + e] = A;
        if (e == 0) {
            mlp[2 * row] = M;
            mlp[2 * row + 1] = L;
        }
    }
}

}  // namespace

int attn_tokens_per_sweep(int d, int nq, int nkv) {
    const int G = nq / nkv;
    if (d == 256 && G == 6) return 2;
    if (d == 64 && (G == 4 || G == 2)) return 4;
    return 1;
}

hipError_t launch_append(const AttnArgs& a, hipStream_t s) {
    if (a.nt < 1 || a.fmt != 0) return hipErrorInvalidValue;
    const dim3 grid(a.nkv, a.nt), block(64);
    if (a.d == 256) hipLaunchKernelGGL(k_append<256>, grid, block, 0, s, a);
    else if (a.d == 64) hipLaunchKernelGGL(k_append<64>, grid, block, 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

// a.nt tokens: one sweep block per attn_tokens_per_sweep tokens (grid z)
hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
    const int G = a.nq / a.nkv;
    if (a.nsplit < 1 || a.nsplit > 256 || a.nt < 1 || (a.nt > 1 && a.append && !a.batch) || a.nq * a.nt > a.prow)
        return hipErrorInvalidValue;
    const int nn = a.nt == 1 || a.batch ? 1 : attn_tokens_per_sweep(a.d, a.nq, a.nkv);
    const int nz = (a.nt + nn - 1) / nn;
    if (a.zfast && (a.batch || nn == 1 || a.append)) return hipErrorInvalidValue;
    const dim3 grid(a.zfast ? a.nsplit * nz : a.nsplit, a.nkv, a.zfast ? 1 : nz), block(64 * kWaves);
    if (a.fmt != 0) {
        // the 4-bit and codebook caches: single-token sweeps of one sequence
        if (a.nt != 1 || a.batch || a.win > 0) return hipErrorInvalidValue;
#define AW4_ATTN_FMT(DD, GG)                                                                  \
        if (a.d == DD && G == GG) {                                                           \
            if (a.fmt == 1) hipLaunchKernelGGL((k_attn<DD, GG, 1, 1>), grid, block, 0, s, a); \
            else if (a.fmt == 2) hipLaunchKernelGGL((k_attn<DD, GG, 1, 2>), grid, block, 0, s, a); \
            else return hipErrorInvalidValue;                                                 \
            return hipGetLastError();                                                         \
        }
        AW4_ATTN_FMT(256, 6)
        AW4_ATTN_FMT(64, 4)
        AW4_ATTN_FMT(64, 2)
#undef AW4_ATTN_FMT
        return hipErrorInvalidValue;
    }
#define AW4_ATTN_CASE(DD, GG, NN)                                               \
    if (a.d == DD && G == GG && nn == NN) {                                     \
        hipLaunchKernelGGL((k_attn<DD, GG, NN>), grid, block, 0, s, a);         \
        return hipGetLastError();                                               \
    }
    AW4_ATTN_CASE(256, 6, 1)
    AW4_ATTN_CASE(256, 6, 2)
    AW4_ATTN_CASE(256, 4, 1)
    AW4_ATTN_CASE(256, 8, 1)
    AW4_ATTN_CASE(256, 2, 1)
    AW4_ATTN_CASE(256, 1, 1)
    AW4_ATTN_CASE(64, 4, 1)
    AW4_ATTN_CASE(64, 4, 4)
    AW4_ATTN_CASE(64, 2, 1)
    AW4_ATTN_CASE(64, 2, 4)
    AW4_ATTN_CASE(64, 1, 1)
    AW4_ATTN_CASE(64, 6, 1)
    AW4_ATTN_CASE(64, 8, 1)
#undef AW4_ATTN_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_attn_win(const AttnArgs& a, hipStream_t s) {
    const int G = a.nq / a.nkv;
    if (a.win < 1 || a.nsplit_w < 1 || a.nt != 1 || a.batch || a.nq > a.prow || !a.kw || !a.vw || a.fmt != 0)
        return hipErrorInvalidValue;
    const dim3 grid(a.nsplit_w, a.nkv), block(64 * kWinWaves);
#define AW4_WIN_CASE(DD, GG)                                            \
    if (a.d == DD && G == GG) {                                         \
        hipLaunchKernelGGL((k_attn_win<DD, GG>), grid, block, 0, s, a); \
        return hipGetLastError();                                       \
    }
    AW4_WIN_CASE(256, 6)
    AW4_WIN_CASE(256, 4)
    AW4_WIN_CASE(256, 2)
    AW4_WIN_CASE(256, 1)
    AW4_WIN_CASE(64, 4)
    AW4_WIN_CASE(64, 2)
    AW4_WIN_CASE(64, 1)
    AW4_WIN_CASE(64, 6)
    AW4_WIN_CASE(64, 8)
#undef AW4_WIN_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
    if (a.nsplit < 1 || a.nsplit + a.nsplit_w > 256) return hipErrorInvalidValue;
    if (a.nt < 1 || a.nq * a.nt > a.prow) return hipErrorInvalidValue;
    // split rows per thread: 16 (D = 256) or 64 (D = 64) rows are in flight
    const int ns = a.nsplit + a.nsplit_w;
    const dim3 grid(a.nq * a.nt), block(1024);
    if (a.d == 256 && a.fmt == 1) {
        // values cached unrotated
        if (ns <= 64) hipLaunchKernelGGL((k_combine<256, 4, false>), grid, block, 0, s, a);
        else if (ns <= 128) hipLaunchKernelGGL((k_combine<256, 8, false>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((k_combine<256, 16, false>), grid, block, 0, s, a);
    } else if (a.d == 256) {
        if (ns <= 64) hipLaunchKernelGGL((k_combine<256, 4>), grid, block, 0, s, a);
        else if (ns <= 128) hipLaunchKernelGGL((k_combine<256, 8>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((k_combine<256, 16>), grid, block, 0, s, a);
    } else if (a.d == 64 && a.fmt == 1) {
        hipLaunchKernelGGL((k_combine<64, 4, false>), grid, block, 0, s, a);
    } else if (a.d == 64) {
        hipLaunchKernelGGL((k_combine<64, 4>), grid, block, 0, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace aw4

// Internal declarations shared by the host runtime and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aw4 {

// Device-resident control block: everything a captured step reads or writes
// that changes from token to token lives here, so one graph serves all steps.
struct Ctl {
    int32_t pos;        // position of the token being decoded
    int32_t token;      // token fed to the next embedding
    int32_t argmax;     // last argmax
    int32_t nstep;      // index into the greedy output ring
    int32_t pad[60];
};

// W4 GPU layout: codes as dwords [rows][cols/8]; within each dword the eight
// 4-bit fields (nibble = code + 8) hold elements [0,2,4,6,1,3,5,7] of its
// 8-element run, so that masks 0x000F000F / 0x00F000F0 (and the same after an
// 8-bit shift) yield element pairs (0,1) (2,3) (4,5) (6,7); scales fp16 bits
// [rows][cols/32].
__host__ __device__ inline int w4_slot(int e) { return (e & 1) ? 4 + (e >> 1) : (e >> 1); }

enum Prologue { PRO_NORM = 0, PRO_GATED = 1, PRO_LOADH = 2 };
enum Epilogue { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2 };

struct GemvArgs {
    const uint32_t* codes;
    const uint16_t* scales;
    int32_t rows;
    int32_t K;
    const float* x;       // NORM: residual [K]; GATED: o [K]
    const float* nw;      // NORM: norm weight [K]; GATED: norm weight [gated_d]
    const float* z;       // GATED: gate input z [K]
    const _Float16* h;    // LOADH: fp16 input [K]
    int32_t gated_d;
    float eps;
    float* y;             // STORE: out [rows]; RESID: residual [rows] (y[r] += dot)
    _Float16* hout;       // SWIGLU: fp16 out [rows/2]; rows interleave gate/up
};

struct HeadArgs {
    const int8_t* codes;      // [V][H]
    const uint16_t* scales;   // [V][H/32]
    int32_t V;
    int32_t H;
    const float* x;           // residual [H]
    const float* nw;          // final norm weight [H]
    float eps;
    float* logits;            // [V] or null
    float* part_val;          // per-block best value
    int32_t* part_idx;        // per-block best index
};

struct GdnArgs {
    const float* proj;        // [q nqk*d | k nqk*d | v nv*d | z nv*d | a nv | b nv]
    const float* a_bias;      // [nv]
    float* S;                 // [nv][d][d]
    float* o;                 // [nv*d]
    int32_t nqk, nv, d;
    float eps;
};

struct AttnArgs {
    const float* proj;        // [q nq*d | g nq*d | k nkv*d | v nkv*d]
    int8_t* kc;               // [nkv][max_ctx][d]
    uint16_t* ks;             // [nkv][max_ctx][d/32]
    uint32_t* vc;             // [nkv][max_ctx][d/32][3] packed 3-bit (value i of a group at bits 3i..3i+2)
    uint16_t* vs;             // [nkv][max_ctx][d/32]
    const float* signs;       // [d] +-1
    const Ctl* ctl;
    float* part;              // [nq][nsplit][d + 2]: acc[d], m, l
    int32_t max_ctx, nq, nkv, d, nsplit;
};

struct CombineArgs {
    const float* part;
    const float* proj;        // for the gate g
    const float* signs;
    const Ctl* ctl;
    _Float16* out;            // [nq*d]
    int32_t nq, nkv, d, nsplit;
};

// ---------------------------------------------------------------- launches
hipError_t launch_gemv(int pro, int epi, const GemvArgs& a, hipStream_t s);
int gemv_blocks(int rows);
hipError_t launch_head(const HeadArgs& a, hipStream_t s);
int head_blocks(int V);
hipError_t launch_head_final(const float* pv, const int32_t* pi, int n, Ctl* ctl, int32_t* ring, int ring_cap,
                             hipStream_t s);
hipError_t launch_gdn(const GdnArgs& a, hipStream_t s);
hipError_t launch_attn(const AttnArgs& a, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_embed(const int8_t* codes, const uint16_t* scales, int H, const Ctl* ctl, float* x,
                        hipStream_t s);
hipError_t launch_set_token(Ctl* ctl, int32_t token, hipStream_t s);
hipError_t launch_advance(Ctl* ctl, hipStream_t s);
hipError_t launch_set_ctl(Ctl* ctl, int32_t pos, int32_t token, int32_t nstep, hipStream_t s);
hipError_t launch_fill_zero(void* p, uint64_t bytes, hipStream_t s);
hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t s);

// quantise fp32 rows into the GPU layouts
hipError_t launch_quant_w4(const float* src, int64_t nrows, int64_t cols, uint32_t* codes, uint16_t* scales,
                           int64_t row_stride, hipStream_t s);
hipError_t launch_quant_i8(const float* src, int64_t nrows, int64_t cols, int8_t* codes, uint16_t* scales,
                           hipStream_t s);

}  // namespace aw4

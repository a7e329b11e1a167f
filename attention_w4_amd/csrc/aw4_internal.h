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
    // draft verification
    int32_t vtok[4];    // t0 (last emitted) and the drafts
    float vu[4];        // uniforms: one per draft, the last for the draw
    float vmax[4];      // max logit per verified position
    float vz[4];        // softmax normaliser per verified position
    int32_t vargmax[4];
    int32_t vout[4];    // emitted tokens
    int32_t vn_acc;     // drafts accepted
    int32_t vn_out;     // tokens emitted (vn_acc + 1)
    int32_t vcommit;    // positions committed (vn_acc + 1)
    int32_t vresid_p;   // 1 when the residual was all zero and p was used
    // draft head
    int32_t dpos;       // committed entries of the draft head's cache
    int32_t dtok[4];    // tokens of the entries a draft call feeds first
    float du[4];        // one uniform per draft
    int32_t dout[4];    // drafts (token ids)
    float dmax;         // largest mapped score of the current draft step
    float dz;           // its softmax normaliser
    int32_t darg;       // index into the map of the current draft
    // batch decode: one token per sequence b, each at its own position
    int32_t btok[4];
    int32_t bpos[4];
    int32_t pad[8];
};
static_assert(sizeof(Ctl) == 256, "control block size");

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

// M input vectors (M <= 4, one per verified token), vectors at fixed strides
struct GemvMultiArgs {
    const uint32_t* codes;
    const uint16_t* scales;
    int32_t rows;
    int32_t K;
    int32_t M;
    const float* x;        // NORM / GATED input, vector m at x + m * sx
    int64_t sx;
    const float* nw;
    const float* z;        // GATED gate input, vector m at z + m * sz
    int64_t sz;
    const _Float16* h;     // LOADH input, vector m at h + m * sh
    int64_t sh;
    int32_t gated_d;
    float eps;
    float* y;              // STORE / RESID output, vector m at y + m * sy
    int64_t sy;
    _Float16* hout;        // SWIGLU output, vector m at hout + m * so
    int64_t so;
};

struct HeadArgs {
    const int8_t* codes;      // [rows][H]
    const uint16_t* scales;   // [rows][H/32]
    const int32_t* map;       // null: output i is row i; else row map[i]
    int32_t V;                // outputs
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
    // grid z > 1 (batch decode): sequence b's token, state and readout at
    // proj + b sproj, S + b sstride, o + b so
    int64_t sproj, sstride, so;
};

struct AttnArgs {
    int32_t pos_offset;       // the first token sits at *pos + pos_offset
    int32_t nt;               // tokens in this sweep, at consecutive positions
    int32_t append;           // encode and append the (single) token first
    int64_t sproj;            // token m's projections at proj + m * sproj
    const float* proj;        // [q nq*d | g nq*d | k nkv*d | v nkv*d]
    int8_t* kc;               // [nkv][max_ctx][d] code + 128, dims permuted for the MFMA operand (k_attn.hip)
    uint16_t* ks;             // [nkv][max_ctx][d/32]
    uint32_t* vc;             // [nkv][max_ctx][3 d/32] 3-bit codes + 4, dims permuted (k_attn.hip)
    uint16_t* vs;             // [nkv][max_ctx][d/32]
    const float* signs;       // [d] +-1
    const int32_t* pos;       // device: the cache's committed length (ctl->pos, or ctl->dpos for the draft head)
    float* part;              // [prow][nsplit][d] acc, then [prow][nsplit][2] (m, l); row m nq + head
    int32_t batch;            // 1: grid z is a sequence: its token at pos[z], its cache at + z seq_bytes
    int64_t seq_bytes;
    int32_t prow;             // rows of part: nq times the most tokens per sweep
    int32_t max_ctx, nq, nkv, d, nsplit;
    // recent window (win > 0): positions [npos - win, npos) are read at fp16
    // from the ring kw/vw ([nkv][win][d], position t at slot t % win) by
    // k_attn_win into split slots nsplit .. nsplit + nsplit_w - 1 of each
    // partial row; k_attn covers the positions before the window
    int32_t win, nsplit_w;
    _Float16* kw;
    _Float16* vw;
    int32_t fmt;              // cache format (k_attn.hip): 0 int8 K + rotated 3-bit V, 1 q4_0, 2 codebook V
    int32_t zfast;            // several token blocks of one sequence: blocks of a split adjacent in dispatch order
};

struct CombineArgs {
    int32_t pos_offset;
    int32_t nt;               // tokens of the sweep (rows m nq + head of part)
    int64_t sproj;            // token m's projections (for the gate g) at proj + m * sproj
    const float* part;
    const float* proj;
    const float* signs;
    const int32_t* pos;
    _Float16* out;            // token m, head h at out + (m nq + h) d
    int32_t prow;
    int32_t nq, nkv, d, nsplit;
    int32_t batch;            // 1: token m is sequence m's single token at pos[m]
    int32_t win, nsplit_w;    // recent window (AttnArgs): the window's splits follow the others
    int32_t fmt;              // cache format: 1 keeps values unrotated
};

struct GdnMultiArgs {
    const float* proj;        // token m's projections at proj + m * sproj
    int64_t sproj;
    const float* a_bias;
    float* S;
    float* o;                 // token m's readout at o + m * so
    int64_t so;
    int32_t nqk, nv, d, M;
    float eps;
    int32_t replay;           // 1: apply *commit_n steps and write S back
    const int32_t* commit_n;
};

// the replay of up to kMaxReplayLayers GDN layers in one launch: common
// fields in a (replay = 1, commit_n set), per-layer inputs and states
constexpr int kMaxReplayLayers = 64;
struct GdnReplayArgs {
    GdnMultiArgs a;
    int32_t nlayers;
    const float* proj[kMaxReplayLayers];
    const float* a_bias[kMaxReplayLayers];
    float* S[kMaxReplayLayers];
};

struct AcceptArgs {
    Ctl* ctl;
    const float* logits;      // [k+1][V]
    const float* q;           // [k][V] draft probabilities (unused when greedy)
    int32_t V, k, greedy;
    float inv_t;
    float* zpart;             // [k+1][nb]
    float* wpart;             // [k+1][nb]
};

// Draft head input of M entries: u_m = [fp16(RMSNorm(emb(tok[m])) * nw_emb);
// fp16(RMSNorm(h_m) * nw_hid)], [M][2H]
struct DraftEmbedArgs {
    const int8_t* codes;      // tied int8 table [V][H]
    const uint16_t* scales;
    const int32_t* tok;       // device token ids [M]
    const float* h;           // hidden m at h + m * sh
    int64_t sh;
    const float* nw_emb;
    const float* nw_hid;
    _Float16* u;              // [M][2H]
    int32_t H, M;
    float eps;
};

// Draft selection from the mapped scores z [Vd] and the head's block partials
struct DraftSelArgs {
    Ctl* ctl;
    const float* z;           // [Vd] mapped scores
    const float* pv;          // head block partials (best value, best index)
    const int32_t* pi;
    int32_t nb;               // head blocks
    const int32_t* map;       // [Vd] ascending ids
    const int32_t* rmap;      // [V] index into the map or -1
    int32_t Vd, V;
    int32_t j;                // draft index
    int32_t commit;           // entries to add to ctl->dpos (the first step) or 0
    int32_t greedy;
    float inv_t;
    float* zpart;             // [draft_chunks(Vd)]
    float* q;                 // [V] draft probabilities of draft j, or null
};

// W4 GEMM of the prefill: Y[m][n] = sum_k X[m][k] W[n][k] over M tokens
struct GemmArgs {
    const uint32_t* codes;   // W4 GPU layout [N][K/8]
    const uint16_t* scales;  // [N][K/32]
    int32_t N, K, M;
    const _Float16* x;       // [M][ldx] fp16 inputs
    int64_t ldx;
    float* y;                // STORE / RESID: [M][ldy]
    int64_t ldy;
    _Float16* hout;          // SWIGLU: [M][ldo], column n / 2 from rows n, n + 1
    int64_t ldo;
    // split-K of the last, partial round of tiles (null part: no split): each
    // split writes its 128 x 128 fp32 partial tile to a slot of part
    // (part_slots slots); a second kernel adds a tile's splits in split order
    // and runs the epilogue
    float* part;
    int32_t part_slots;
    int32_t nfull, nsplit;   // set by the launcher: units [0, nfull) are whole tiles
};

// Gated DeltaNet over the T tokens of a prefill chunk
struct GdnPrefillArgs {
    const float* proj;       // token t's projections at proj + t * sproj
    int64_t sproj;
    const float* a_bias;
    float* S;                // [nv][d][d], read at the start, written at the end
    float* qn;               // [T][nqk][d] normalised q
    float* kn;               // [T][nqk][d] normalised k
    float* ab;               // [T][nv][2] alpha, beta
    float* o;                // token t's readout at o + t * so
    int64_t so;
    int32_t nqk, nv, d, T;
    float eps;
};

// ---------------------------------------------------------------- launches
hipError_t launch_gemv(int pro, int epi, const GemvArgs& a, hipStream_t s);
int gemv_blocks(int rows);
hipError_t launch_head(const HeadArgs& a, hipStream_t s);
hipError_t launch_gemv_multi(int pro, int epi, const GemvMultiArgs& a, hipStream_t s);
// int8 head over M vectors: logits [M][V], per-block best per vector [M][nblocks]
struct HeadMultiArgs {
    const int8_t* codes;
    const uint16_t* scales;
    int32_t V, H, M;
    const float* x;        // residuals, vector m at x + m * H
    const float* nw;
    float eps;
    float* logits;         // [M][V]
    float* part_val;       // [M][nparts]
    int32_t* part_idx;
    int32_t nparts;        // partial slots per vector (set by launch_head_multi: head_blocks(V))
};
hipError_t launch_head_multi(const HeadMultiArgs& a, hipStream_t s);
int head_blocks(int V);
// workgroups of 256 threads of fn (shm bytes of dynamic LDS) resident at once
int resident_blocks(const void* fn, size_t shm);
int draft_head_blocks(int V);   // blocks of the mapped head (launch_head with a map)
hipError_t launch_head_final(const float* pv, const int32_t* pi, int n, Ctl* ctl, int32_t* ring, int ring_cap,
                             hipStream_t s);
hipError_t launch_gdn(const GdnArgs& a, hipStream_t s);
hipError_t launch_gdn_batch(const GdnArgs& a, int B, hipStream_t s);
hipError_t launch_gdn_multi(const GdnMultiArgs& a, hipStream_t s);
hipError_t launch_gdn_replay(const GdnReplayArgs& r, hipStream_t s);
int accept_blocks(int V);
hipError_t launch_accept(const AcceptArgs& a, const float* head_pv, const int32_t* head_pi, int head_nb,
                         hipStream_t s);
hipError_t launch_commit_pos(Ctl* ctl, hipStream_t s);
hipError_t launch_embed_tokens(const int8_t* codes, const uint16_t* scales, int H, const int32_t* tok, int M, float* x,
                               hipStream_t s);
hipError_t launch_set_batch(Ctl* ctl, const int32_t* tok, const int32_t* pos, hipStream_t s);
// per-vector best value and index from the head's block partials into ctl->vmax / vargmax
hipError_t launch_head_argmax_multi(const float* pv, const int32_t* pi, int nb, int M, Ctl* ctl, hipStream_t s);
hipError_t launch_embed_multi(const int8_t* codes, const uint16_t* scales, int H, const Ctl* ctl, int M, float* x,
                              hipStream_t s);
hipError_t launch_set_verify(Ctl* ctl, const int32_t* tok, const float* u, hipStream_t s);
hipError_t launch_attn(const AttnArgs& a, hipStream_t s);
hipError_t launch_append(const AttnArgs& a, hipStream_t s);
int attn_tokens_per_sweep(int d, int nq, int nkv);
hipError_t launch_attn_win(const AttnArgs& a, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_embed(const int8_t* codes, const uint16_t* scales, int H, const Ctl* ctl, float* x,
                        hipStream_t s);
hipError_t launch_set_token(Ctl* ctl, int32_t token, hipStream_t s);
hipError_t launch_advance(Ctl* ctl, hipStream_t s);
hipError_t launch_set_ctl(Ctl* ctl, int32_t pos, int32_t token, int32_t nstep, hipStream_t s);
hipError_t launch_fill_zero(void* p, uint64_t bytes, hipStream_t s);
hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t s);
// plain streaming read of bytes (a multiple of 16) by nblocks workgroups; sink [nblocks]
hipError_t launch_stream_read(const void* src, uint64_t bytes, uint32_t* sink, int nblocks, hipStream_t s);
hipError_t launch_draft_embed(const DraftEmbedArgs& a, hipStream_t s);
hipError_t launch_draft_select(const DraftSelArgs& a, hipStream_t s);
int draft_chunks(int Vd);
hipError_t launch_set_draft(Ctl* ctl, const int32_t* tok, const float* u, hipStream_t s);
hipError_t launch_set_dpos(Ctl* ctl, int32_t dpos, hipStream_t s);
hipError_t launch_gemm_w4(int epi, const GemmArgs& a, hipStream_t s);
hipError_t launch_embed_rows(const int8_t* codes, const uint16_t* scales, int H, const int32_t* tok, int T, float* x,
                             hipStream_t s);
hipError_t launch_norm_rows(const float* x, const float* w, int K, float eps, int T, _Float16* out, int64_t ldo,
                            hipStream_t s);
// normalised q, k and gates, the recurrence, then fp16(RMSNorm(o) w SiLU(z)) into out [T][ldo]
hipError_t launch_gdn_prefill(const GdnPrefillArgs& a, const float* gated_w, _Float16* out, int64_t ldo,
                              hipStream_t s);

// quantise fp32 rows into the GPU layouts
hipError_t launch_quant_w4(const float* src, int64_t nrows, int64_t cols, uint32_t* codes, uint16_t* scales,
                           int64_t row_stride, hipStream_t s);
hipError_t launch_quant_i8(const float* src, int64_t nrows, int64_t cols, int8_t* codes, uint16_t* scales,
                           hipStream_t s);

}  // namespace aw4

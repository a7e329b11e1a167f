// Host runtime behind the C ABI in include/aw4.h: config validation, arena
// planning, weight packing/export, the per-token launch sequence and its HIP
// graph, and state import/export.  All device memory comes from the caller's
// arena; nothing here allocates device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/aw4.h"
#include "aw4_internal.h"

using namespace aw4;

namespace {

struct LayerBufs {
    char type = 'G';
    int64_t in_rows = 0, out_cols = 0;
    uint32_t* w_in = nullptr;
    uint16_t* s_in = nullptr;
    uint32_t* w_out = nullptr;
    uint16_t* s_out = nullptr;
    uint32_t* w_gu = nullptr;   // gate/up interleaved: row 2i gate i, row 2i+1 up i
    uint16_t* s_gu = nullptr;
    uint32_t* w_down = nullptr;
    uint16_t* s_down = nullptr;
    float* norm_mix = nullptr;
    float* norm_ffn = nullptr;
    float* norm_gated = nullptr;
    float* a_bias = nullptr;
    float* S = nullptr;
    int8_t* kc = nullptr;
    uint16_t* ks = nullptr;
    uint32_t* vc = nullptr;
    uint16_t* vs = nullptr;
    _Float16* kw = nullptr;     // recent window (kv_window > 0): fp16 keys [nkv][W][d], slot t % W
    _Float16* vw = nullptr;     // fp16 rotated values, same slots
};

// one tensor of a config and the rows of it that have been set
struct TensorSlot {
    int layer = 0, kind = 0;
    int64_t rows = 0;
    std::vector<bool> done;
    int64_t ndone = 0;
};

constexpr int kSweepRows = 4;   // most tokens one attention sweep takes (verify_k has at most 4)
constexpr int kPrefillMaxChunk = 1024;   // prompt tokens per prefill chunk (buffers sized for it)
constexpr int kGemmSplitSlots = 512;     // split-K partial tiles of the chunk GEMM (64 KB each)

struct Plan {
    uint64_t off = 0;
    uint8_t* base = nullptr;   // null while only sizing
    template <class T>
    T* take(uint64_t bytes) {
        off = (off + 255) & ~uint64_t(255);
        T* p = base ? (T*)(base + off) : nullptr;
        off += bytes;
        return p;
    }
};

}  // namespace

struct aw4_model {
    aw4_config cfg{};
    uint8_t* arena = nullptr;
    uint64_t arena_bytes = 0;
    hipStream_t stream = nullptr;
    std::vector<LayerBufs> L;
    int8_t* lm_codes = nullptr;
    uint16_t* lm_scales = nullptr;
    float* norm_final = nullptr;
    float* signs = nullptr;
    Ctl* ctl = nullptr;
    float* x = nullptr;
    float* proj = nullptr;
    float* obuf = nullptr;
    _Float16* hbuf = nullptr;
    _Float16* abuf = nullptr;
    float* part = nullptr;
    float* logits = nullptr;
    float* pv = nullptr;
    int32_t* pi = nullptr;
    int32_t* ring = nullptr;
    int ring_cap = 0;
    // draft verification (M = k + 1 tokens)
    float* vx = nullptr;            // [max_verify][H] residuals
    std::vector<float*> vproj_g;    // per GDN layer [max_verify][in_rows] (kept for the replay)
    float* vproj_a = nullptr;       // [max_verify][attn in_rows]
    float* vo = nullptr;            // [max_verify][nv*d]
    _Float16* vh = nullptr;         // [max_verify][hlen]
    _Float16* va = nullptr;         // [max_verify][nq*dh]
    float* vlogits = nullptr;       // [max_verify][V]
    float* vpv = nullptr;           // [max_verify][nhb]
    int32_t* vpi = nullptr;
    float* vzpart = nullptr;        // [max_verify][accept blocks]
    float* vwpart = nullptr;
    int64_t hlen = 0;
    int nhead_blocks = 0;
    int nsplit = 1;
    int nsplit_w = 0;               // splits of the recent window's sweep (kv_window > 0)
    int32_t host_pos = 0;
    // draft head (draft_vocab > 0)
    LayerBufs D;                    // its gated-attention layer; cache in the state region
    uint32_t* w_fuse = nullptr;     // [H][2H] W4
    uint16_t* s_fuse = nullptr;
    float* dn_emb = nullptr;
    float* dn_hid = nullptr;
    float* dn_out = nullptr;
    int32_t* dmap = nullptr;        // [draft_vocab] ascending ids
    int32_t* drmap = nullptr;       // [vocab] index into dmap or -1
    float* xd = nullptr;            // [max_verify][H] the draft block's residuals
    _Float16* ubuf = nullptr;       // [max_verify][2H] its fp16 inputs
    float* dscore = nullptr;        // [draft_vocab] mapped scores of the current step
    float* dpv = nullptr;           // head block partials
    int32_t* dpi = nullptr;
    float* dzpart = nullptr;        // [draft chunks]
    int ndhead_blocks = 0;
    bool map_set = false;
    int32_t host_dpos = 0;
    // what the next draft call feeds before its own entry: the hidden rows of
    // the committed positions (none, the decode residual, or verify rows) and
    // the tokens that followed them
    int pend_src = 0;               // 0 nothing to draft from, 1 x, 2 vx rows 0..pend_n
    int pend_n = 0;
    int32_t pend_tok[4] = {0, 0, 0, 0};
    // prefill chunk buffers (C = pchunk_max tokens)
    int pchunk_max = 0;             // 0: no chunked prefill (shapes the GEMM does not take)
    int pchunk = 0;                 // current chunk size (aw4_set_prefill_chunk), 0: token by token
    int32_t* ptok = nullptr;        // [C] token ids
    int32_t* pnext = nullptr;       // [C] the next token of each (draft head entries)
    float* px = nullptr;            // [C][H] residuals
    _Float16* pa = nullptr;         // [C][pa_ld] fp16 GEMM inputs
    int64_t pa_ld = 0;
    _Float16* pf = nullptr;         // [C][F] SwiGLU outputs
    float* pp = nullptr;            // [C][max_in] projections
    float* po = nullptr;            // [C][nv d] GDN readouts
    float* pqn = nullptr;           // [C][nqk d]
    float* pkn = nullptr;
    float* pab = nullptr;           // [C][nv][2]
    float* ppart = nullptr;         // attention partials, one split: [C nq][d + 2]
    float* gpart = nullptr;         // chunk GEMM split-K partial tiles [kGemmSplitSlots][128 x 128]
    uint64_t state_off = 0, state_bytes = 0;   // recurrent states + caches of one sequence
    // sequences: max_batch copies of the state region, state_bytes apart; the
    // single-sequence calls work on sequence `seq` (aw4_select_sequence)
    int max_batch = 1;
    int seq = 0;
    int32_t seq_pos[4] = {0, 0, 0, 0};
    int32_t seq_dpos[4] = {0, 0, 0, 0};
    // which tensors have been given values (quantize/load/set calls and
    // aw4_load_weights): the model computes only once every tensor of its
    // config is complete
    std::vector<TensorSlot> slots;
    int slots_missing = 0;
    // recent window: false for a layer whose ring may hold entries of positions
    // after the current one (set_pos moved back; aw4_import_state_win refreshes
    // it); win_imported: the ring was imported since the last decode call, so it
    // describes whatever position the caller sets next
    std::vector<bool> win_fresh, win_imported;
    // split partials of the single-token step's attention sweeps (rows of one
    // token) and the output head's block partials: the arena's by default,
    // the library's static scratch inside aw4_decode_step_static
    float* step_part = nullptr;
    int step_prow = 0;
    float* step_pv = nullptr;
    int32_t* step_pi = nullptr;
    uint8_t* static_scratch = nullptr;   // this device's static scratch (hipGetSymbolAddress)
    uint64_t static_need = 0;            // bytes of it the step needs
    bool use_graph = true;
    hipGraphExec_t g_head = nullptr;
    hipGraphExec_t g_nohead = nullptr;
    hipGraphExec_t g_batch[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};   // per batch size
    std::string err;
};

namespace {

const int kRingCap = 1 << 16;

int fail(aw4_model* m, int code, const std::string& msg) {
    if (m) m->err = msg;
    return code;
}

// Failure injection for tests of the error path: when armed with n >= 1, the
// n-th checked HIP call from then on reports hipErrorUnknown (the call itself
// has run), once.  Calls that open a stream capture are not counted, so an
// injected failure never leaves a capture open.
std::atomic<int> g_fail_countdown{0};

hipError_t counted(hipError_t e) {
    if (e != hipSuccess) return e;
    int n = g_fail_countdown.load(std::memory_order_relaxed);
    while (n > 0 && !g_fail_countdown.compare_exchange_weak(n, n - 1, std::memory_order_relaxed)) {
    }
    return n == 1 ? hipErrorUnknown : hipSuccess;
}

#define HIPCHK(m, expr)                                                                        \
    do {                                                                                       \
        hipError_t e_ = counted(expr);                                                         \
        if (e_ != hipSuccess)                                                                  \
            return fail((m), AW4_E_HIP, std::string(#expr) + ": " + hipGetErrorString(e_));    \
    } while (0)

// the same without the injection count (calls that begin a stream capture)
#define HIPCHK_RAW(m, expr)                                                                    \
    do {                                                                                       \
        hipError_t e_ = (expr);                                                                \
        if (e_ != hipSuccess)                                                                  \
            return fail((m), AW4_E_HIP, std::string(#expr) + ": " + hipGetErrorString(e_));    \
    } while (0)

int64_t mix_in_rows(const aw4_config* c, char t) {
    if (t == 'G')
        return 2LL * c->gdn_qk_heads * c->gdn_head_dim + 2LL * c->gdn_v_heads * c->gdn_head_dim +
               2LL * c->gdn_v_heads;
    return 2LL * c->attn_q_heads * c->attn_head_dim + 2LL * c->attn_kv_heads * c->attn_head_dim;
}

int64_t mix_out_cols(const aw4_config* c, char t) {
    return t == 'G' ? (int64_t)c->gdn_v_heads * c->gdn_head_dim : (int64_t)c->attn_q_heads * c->attn_head_dim;
}

// Cache row layouts written and read by k_attn.hip: the key code + 128 of
// logical dim e of a row of d bytes sits at byte kv_key_byte(e, d); the 3-bit
// field (code + 4) of logical value dim e starts at bit kv_value_bit(e, d) of the
// position's record.
int kv_key_byte(int e, int d) { return 8 * (d / 32) * ((e & 31) >> 3) + 8 * (e >> 5) + (e & 7); }
int kv_value_bit(int e, int d) { return 3 * ((d / 16) * (e & 15) + (e >> 4)); }
// 4-bit keys (kv_format 1): logical dim e = 32 g + 8 q + i is the nibble (code
// + 8) at slot [0,2,4,6,1,3,5,7][i] of dword q (d/32) + g of the row
int kv_key_nib_bit(int e, int d) { return 32 * (((e & 31) >> 3) * (d / 32) + (e >> 5)) + 4 * w4_slot(e & 7); }
// value fields of FB bits: logical dim e's field starts at FB ((d/16)(e % 16) + e / 16)
int kv_value_bit_fb(int e, int d, int fb) { return fb * ((d / 16) * (e & 15) + (e >> 4)); }
// codebook indices 0..7 (ascending levels) <-> sign-magnitude fields (bit 2: negative)
uint32_t lm_field(int c) { return c >= 4 ? (uint32_t)(c - 4) : (uint32_t)(7 - c); }
int lm_code(uint32_t f) { return (f & 4) ? 7 - (int)f : (int)f + 4; }

uint32_t kv_value_field(const uint32_t* rec, int words, int bit) {
    const int wi = bit >> 5, off = bit & 31;
    uint64_t x = rec[wi];
    if (wi + 1 < words) x |= (uint64_t)rec[wi + 1] << 32;
    return (uint32_t)(x >> off) & 7u;
}

uint32_t kv_value_field(const uint32_t* rec, int words, int bit, int fb) {
    const int wi = bit >> 5, off = bit & 31;
    uint64_t x = rec[wi];
    if (wi + 1 < words) x |= (uint64_t)rec[wi + 1] << 32;
    return (uint32_t)(x >> off) & ((1u << fb) - 1u);
}

// Splits of the recent window's sweep per kv head: about 64 positions each, at
// most 64 (the window's kernel runs after the main sweep, on its own round).
int win_splits(int win) {
    int n = (win + 63) / 64;
    return n < 1 ? 1 : n > 64 ? 64 : n;
}

// Splits of the attention grid per kv head: one workgroup per compute unit in
// one round (256 units on gfx950; aw4_create lowers it to the device's count),
// never more than there are 16-position tiles of capacity.  The combine merges
// at most 256 split slots per row, the recent window's included.
int nsplit_for(int max_ctx, int nkv, int nsplit_w, int cus = 256) {
    int n = cus / (nkv > 0 ? nkv : 1);
    const int tiles = (max_ctx + 15) / 16;
    if (n > tiles) n = tiles;
    if (n > 256 - nsplit_w) n = 256 - nsplit_w;
    if (n < 1) n = 1;
    return n;
}

// Lays out every buffer in the arena (base null: sizing only).
uint64_t plan_layout(const aw4_config* c, aw4_model* m, uint8_t* base) {
    Plan p;
    p.base = base;
    const int64_t H = c->hidden, F = c->ffn;
    auto w4 = [&](int64_t rows, int64_t cols, uint32_t** w, uint16_t** s) {
        *w = p.take<uint32_t>((uint64_t)rows * cols / 2);
        *s = p.take<uint16_t>((uint64_t)rows * (cols / 32) * 2);
    };
    std::vector<LayerBufs> L(c->n_layers);
    int64_t max_in = 0;
    bool has_g = false, has_a = false;
    for (int l = 0; l < c->n_layers; ++l) {
        LayerBufs& b = L[l];
        b.type = c->layer_pattern[l];
        b.in_rows = mix_in_rows(c, b.type);
        b.out_cols = mix_out_cols(c, b.type);
        if (b.in_rows > max_in) max_in = b.in_rows;
        w4(b.in_rows, H, &b.w_in, &b.s_in);
        w4(H, b.out_cols, &b.w_out, &b.s_out);
        w4(2 * F, H, &b.w_gu, &b.s_gu);
        w4(H, F, &b.w_down, &b.s_down);
        b.norm_mix = p.take<float>(H * 4);
        b.norm_ffn = p.take<float>(H * 4);
        if (b.type == 'G') {
            has_g = true;
            b.norm_gated = p.take<float>((uint64_t)c->gdn_head_dim * 4);
            b.a_bias = p.take<float>((uint64_t)c->gdn_v_heads * 4);
        } else {
            has_a = true;
        }
    }
    int8_t* lm_codes = nullptr;
    uint16_t* lm_scales = nullptr;
    float* norm_final = nullptr;
    if (c->vocab > 0) {
        lm_codes = p.take<int8_t>((uint64_t)c->vocab * H);
        lm_scales = p.take<uint16_t>((uint64_t)c->vocab * (H / 32) * 2);
        norm_final = p.take<float>(H * 4);
    }
    const bool dh = c->draft_vocab > 0;
    float* signs = p.take<float>((uint64_t)(has_a || dh ? c->attn_head_dim : 1) * 4);
    LayerBufs D;
    uint32_t* w_fuse = nullptr;
    uint16_t* s_fuse = nullptr;
    float *dn_emb = nullptr, *dn_hid = nullptr, *dn_out = nullptr;
    int32_t *dmap = nullptr, *drmap = nullptr;
    if (dh) {
        D.type = 'A';
        D.in_rows = mix_in_rows(c, 'A');
        D.out_cols = mix_out_cols(c, 'A');
        if (D.in_rows > max_in) max_in = D.in_rows;
        w4(D.in_rows, H, &D.w_in, &D.s_in);
        w4(H, D.out_cols, &D.w_out, &D.s_out);
        w4(2 * F, H, &D.w_gu, &D.s_gu);
        w4(H, F, &D.w_down, &D.s_down);
        D.norm_mix = p.take<float>(H * 4);
        D.norm_ffn = p.take<float>(H * 4);
        w4(H, 2 * H, &w_fuse, &s_fuse);
        dn_emb = p.take<float>(H * 4);
        dn_hid = p.take<float>(H * 4);
        dn_out = p.take<float>(H * 4);
        dmap = p.take<int32_t>((uint64_t)c->draft_vocab * 4);
        drmap = p.take<int32_t>((uint64_t)c->vocab * 4);
    }
    // recurrent states and caches: one contiguous region, cleared by reset
    p.off = (p.off + 255) & ~uint64_t(255);
    const uint64_t state_off = p.off;
    for (int l = 0; l < c->n_layers; ++l) {
        LayerBufs& b = L[l];
        if (b.type == 'G') {
            b.S = p.take<float>((uint64_t)c->gdn_v_heads * c->gdn_head_dim * c->gdn_head_dim * 4);
        } else {
            // keys: 1 byte per dim (4-bit cache: half); values: 3 (4) bits per dim
            const uint64_t n = (uint64_t)c->attn_kv_heads * c->max_ctx * c->attn_head_dim;
            const bool q4 = c->kv_format == 1;
            b.kc = p.take<int8_t>(q4 ? n / 2 : n);
            b.ks = p.take<uint16_t>(n / 32 * 2);
            b.vc = p.take<uint32_t>(n / 32 * (q4 ? 16 : 12));
            b.vs = p.take<uint16_t>(n / 32 * 2);
            if (c->kv_window > 0) {
                const uint64_t nw = (uint64_t)c->attn_kv_heads * c->kv_window * c->attn_head_dim;
                b.kw = p.take<_Float16>(nw * 2);
                b.vw = p.take<_Float16>(nw * 2);
            }
        }
    }
    if (dh) {
        const uint64_t n = (uint64_t)c->attn_kv_heads * c->max_ctx * c->attn_head_dim;
        D.kc = p.take<int8_t>(n);
        D.ks = p.take<uint16_t>(n / 32 * 2);
        D.vc = p.take<uint32_t>(n / 32 * 12);
        D.vs = p.take<uint16_t>(n / 32 * 2);
    }
    p.off = (p.off + 255) & ~uint64_t(255);
    const uint64_t state_bytes = p.off - state_off;
    const int nbatch = c->max_batch > 1 ? c->max_batch : 1;
    p.off += (uint64_t)(nbatch - 1) * state_bytes;   // the other sequences' copies
    Ctl* ctl = p.take<Ctl>(sizeof(Ctl));
    float* x = p.take<float>(H * 4);
    float* proj = p.take<float>((uint64_t)max_in * 4);
    float* obuf = p.take<float>((uint64_t)(has_g ? c->gdn_v_heads * c->gdn_head_dim : 1) * 4);
    const int64_t hlen = F > (int64_t)c->attn_q_heads * c->attn_head_dim ? F : (int64_t)c->attn_q_heads * c->attn_head_dim;
    // (hlen also sizes the per-token FFN buffers of the verify pass)
    _Float16* hbuf = p.take<_Float16>((uint64_t)hlen * 2);
    _Float16* abuf = p.take<_Float16>((uint64_t)(has_a || dh ? c->attn_q_heads * c->attn_head_dim : 1) * 2);
    const int nsplit_w = c->kv_window > 0 ? win_splits(c->kv_window) : 0;
    const int nsplit = nsplit_for(c->max_ctx, c->attn_kv_heads, nsplit_w);
    // split partials: one row per (token of a sweep, q head), up to 4 tokens,
    // nsplit slots (+ nsplit_w for the recent window) each
    float* part = p.take<float>((uint64_t)(has_a || dh ? kSweepRows * c->attn_q_heads : 1) * (nsplit + nsplit_w) *
                                (c->attn_head_dim + 2) * 4);
    float* logits = nullptr;
    float* pv = nullptr;
    int32_t* pi = nullptr;
    int nhb = 0;
    if (c->vocab > 0) {
        logits = p.take<float>((uint64_t)c->vocab * 4);
        nhb = head_blocks(c->vocab);
        pv = p.take<float>((uint64_t)nhb * 4);
        pi = p.take<int32_t>((uint64_t)nhb * 4);
    }
    int32_t* ring = p.take<int32_t>((uint64_t)kRingCap * 4);
    const int MV = std::max(c->max_verify, c->max_batch);
    float* vx = p.take<float>((uint64_t)MV * H * 4);
    std::vector<float*> vproj_g;
    float* vproj_a = nullptr;
    for (int l = 0; l < c->n_layers; ++l)
        if (L[l].type == 'G') vproj_g.push_back(p.take<float>((uint64_t)MV * L[l].in_rows * 4));
    if (has_a || dh) vproj_a = p.take<float>((uint64_t)MV * mix_in_rows(c, 'A') * 4);
    float* vo = p.take<float>((uint64_t)MV * (has_g ? c->gdn_v_heads * c->gdn_head_dim : 1) * 4);
    _Float16* vh = p.take<_Float16>((uint64_t)MV * hlen * 2);
    _Float16* va = p.take<_Float16>((uint64_t)MV * (has_a || dh ? c->attn_q_heads * c->attn_head_dim : 1) * 2);
    float *vlogits = nullptr, *vpv = nullptr, *vzpart = nullptr, *vwpart = nullptr;
    int32_t* vpi = nullptr;
    if (c->vocab > 0) {
        vlogits = p.take<float>((uint64_t)MV * c->vocab * 4);
        vpv = p.take<float>((uint64_t)MV * nhb * 4);
        vpi = p.take<int32_t>((uint64_t)MV * nhb * 4);
        vzpart = p.take<float>((uint64_t)MV * accept_blocks(c->vocab) * 4);
        vwpart = p.take<float>((uint64_t)MV * accept_blocks(c->vocab) * 4);
    }
    // prefill chunk buffers, when every GEMM row length is a multiple of 64
    const int64_t nvd = (int64_t)c->gdn_v_heads * c->gdn_head_dim, nqd = (int64_t)c->attn_q_heads * c->attn_head_dim;
    bool gemm_ok = c->vocab > 0 && H % 64 == 0 && F % 64 == 0 && (!has_g || nvd % 64 == 0) &&
                   (!(has_a || dh) || nqd % 64 == 0);
    const int C = gemm_ok ? (int)std::min<int64_t>(kPrefillMaxChunk, c->max_ctx) : 0;
    int32_t *ptok = nullptr, *pnext = nullptr;
    float *px = nullptr, *pp = nullptr, *po = nullptr, *pqn = nullptr, *pkn = nullptr, *pab = nullptr, *ppart = nullptr;
    float* gpart = nullptr;
    _Float16 *pa = nullptr, *pf = nullptr;
    int64_t pa_ld = 0;
    if (C > 0) {
        pa_ld = std::max<int64_t>(H, std::max(has_g ? nvd : 0, has_a || dh ? nqd : 0));
        if (dh) pa_ld = std::max<int64_t>(pa_ld, 2 * H);
        ptok = p.take<int32_t>((uint64_t)C * 4);
        pnext = p.take<int32_t>((uint64_t)C * 4);
        px = p.take<float>((uint64_t)C * H * 4);
        pa = p.take<_Float16>((uint64_t)C * pa_ld * 2);
        pf = p.take<_Float16>((uint64_t)C * F * 2);
        pp = p.take<float>((uint64_t)C * max_in * 4);
        if (has_g) {
            po = p.take<float>((uint64_t)C * nvd * 4);
            pqn = p.take<float>((uint64_t)C * c->gdn_qk_heads * c->gdn_head_dim * 4);
            pkn = p.take<float>((uint64_t)C * c->gdn_qk_heads * c->gdn_head_dim * 4);
            pab = p.take<float>((uint64_t)C * c->gdn_v_heads * 2 * 4);
        }
        if (has_a || dh) ppart = p.take<float>((uint64_t)C * c->attn_q_heads * (c->attn_head_dim + 2) * 4);
        gpart = p.take<float>((uint64_t)kGemmSplitSlots * 128 * 128 * 4);
    }
    float *xd = nullptr, *dscore = nullptr, *dpv = nullptr, *dzpart = nullptr;
    _Float16* ubuf = nullptr;
    int32_t* dpi = nullptr;
    int ndhb = 0;
    if (dh) {
        xd = p.take<float>((uint64_t)MV * H * 4);
        ubuf = p.take<_Float16>((uint64_t)MV * 2 * H * 2);
        dscore = p.take<float>((uint64_t)c->draft_vocab * 4);
        ndhb = draft_head_blocks(c->draft_vocab);
        dpv = p.take<float>((uint64_t)ndhb * 4);
        dpi = p.take<int32_t>((uint64_t)ndhb * 4);
        dzpart = p.take<float>((uint64_t)draft_chunks(c->draft_vocab) * 4);
    }
    p.off = (p.off + 255) & ~uint64_t(255);
    if (m) {
        m->pchunk_max = m->pchunk = C;
        m->ptok = ptok;
        m->pnext = pnext;
        m->px = px;
        m->pa = pa;
        m->pa_ld = pa_ld;
        m->pf = pf;
        m->pp = pp;
        m->po = po;
        m->pqn = pqn;
        m->pkn = pkn;
        m->pab = pab;
        m->ppart = ppart;
        m->gpart = gpart;
        m->D = D;
        m->w_fuse = w_fuse;
        m->s_fuse = s_fuse;
        m->dn_emb = dn_emb;
        m->dn_hid = dn_hid;
        m->dn_out = dn_out;
        m->dmap = dmap;
        m->drmap = drmap;
        m->xd = xd;
        m->ubuf = ubuf;
        m->dscore = dscore;
        m->dpv = dpv;
        m->dpi = dpi;
        m->dzpart = dzpart;
        m->ndhead_blocks = ndhb;
        m->vx = vx;
        m->vproj_g = vproj_g;
        m->vproj_a = vproj_a;
        m->vo = vo;
        m->vh = vh;
        m->va = va;
        m->vlogits = vlogits;
        m->vpv = vpv;
        m->vpi = vpi;
        m->vzpart = vzpart;
        m->vwpart = vwpart;
        m->hlen = hlen;
        m->L = L;
        m->lm_codes = lm_codes;
        m->lm_scales = lm_scales;
        m->norm_final = norm_final;
        m->signs = signs;
        m->ctl = ctl;
        m->x = x;
        m->proj = proj;
        m->obuf = obuf;
        m->hbuf = hbuf;
        m->abuf = abuf;
        m->part = part;
        m->step_part = part;
        m->step_prow = kSweepRows * c->attn_q_heads;
        m->logits = logits;
        m->pv = pv;
        m->pi = pi;
        m->step_pv = pv;
        m->step_pi = pi;
        m->ring = ring;
        m->ring_cap = kRingCap;
        m->nhead_blocks = nhb;
        m->nsplit = nsplit;
        m->nsplit_w = nsplit_w;
        // prefill runs token by token with a recent window or the 4-bit and codebook caches
        if (c->kv_window > 0 || c->kv_format != 0) m->pchunk_max = m->pchunk = 0;
        m->state_off = state_off;
        m->state_bytes = state_bytes;
        m->max_batch = nbatch;
    }
    return p.off;
}

const char* check_config(const aw4_config* c) {
    if (!c) return "null config";
    if (c->hidden <= 0 || c->hidden % 64) return "hidden must be a positive multiple of 64";
    if (c->ffn <= 0 || c->ffn % 64) return "ffn must be a positive multiple of 64";
    if (c->group != 32) return "group must be 32";
    if (c->n_layers < 1 || c->n_layers > 127) return "n_layers must be in [1, 127]";
    if ((int)strnlen(c->layer_pattern, 128) != c->n_layers) return "layer_pattern length must equal n_layers";
    bool g = false, a = false;
    for (int i = 0; i < c->n_layers; ++i) {
        if (c->layer_pattern[i] == 'G') g = true;
        else if (c->layer_pattern[i] == 'A') a = true;
        else return "layer_pattern letters must be 'G' or 'A'";
    }
    if (c->draft_vocab < 0) return "draft_vocab must be >= 0";
    if (c->draft_vocab > 0) {
        if (c->vocab <= 0 || c->draft_vocab > c->vocab) return "draft_vocab must be in [0, vocab]";
        a = true;   // the draft head's block has the attention layers' shape
    }
    if (g) {
        if (c->gdn_head_dim != 64 && c->gdn_head_dim != 128) return "gdn_head_dim must be 64 or 128";
        if (c->gdn_qk_heads < 1 || c->gdn_v_heads < 1 || c->gdn_v_heads % c->gdn_qk_heads)
            return "gdn_v_heads must be a positive multiple of gdn_qk_heads";
        if (((int64_t)c->gdn_v_heads * c->gdn_head_dim) % 64) return "gdn_v_heads * gdn_head_dim must be a multiple of 64";
    }
    if (a) {
        if (c->attn_head_dim != 64 && c->attn_head_dim != 256) return "attn_head_dim must be 64 or 256";
        if (c->attn_kv_heads < 1 || c->attn_q_heads < 1 || c->attn_q_heads % c->attn_kv_heads)
            return "attn_q_heads must be a positive multiple of attn_kv_heads";
        const int G = c->attn_q_heads / c->attn_kv_heads;
        if (!(G == 1 || G == 2 || G == 4 || G == 6 || G == 8)) return "attn_q_heads / attn_kv_heads must be 1, 2, 4, 6 or 8";
    }
    if (c->vocab < 0 || c->vocab > (1 << 21)) return "vocab must be in [0, 2097152]";
    if (c->draft_vocab > 0 && c->hidden > 8192) return "hidden must be <= 8192 with a draft head";
    if (c->max_ctx < 1) return "max_ctx must be >= 1";
    if (c->max_verify < 1 || c->max_verify > 4) return "max_verify must be in [1, 4]";
    if (c->max_batch < 0 || c->max_batch > 4) return "max_batch must be in [0, 4]";
    if (c->kv_window < 0 || c->kv_window > c->max_ctx) return "kv_window must be in [0, max_ctx]";
    if (c->kv_window > 0 && (c->max_batch > 1 || c->draft_vocab > 0))
        return "kv_window needs max_batch <= 1 and no draft head (single-sequence decode only)";
    if (c->kv_format < 0 || c->kv_format > 2) return "kv_format must be 0, 1 or 2";
    if (c->kv_format != 0 && (c->kv_window > 0 || c->max_batch > 1 || c->draft_vocab > 0))
        return "kv_format 1 and 2 need no recent window, max_batch <= 1 and no draft head";
    if (!(c->rms_eps > 0.f) || !std::isfinite(c->rms_eps)) return "rms_eps must be positive";
    return nullptr;
}

// host-side nibble permutation between the logical W4 format and the GPU layout
void w4_logical_to_gpu(const uint8_t* src, int64_t cols, uint32_t* dst) {
    for (int64_t d = 0; d < cols / 8; ++d) {
        uint32_t w = 0;
        for (int e = 0; e < 8; ++e) {
            const int64_t k = d * 8 + e;
            const uint32_t nib = (k & 1) ? (src[k >> 1] >> 4) : (src[k >> 1] & 15);
            w |= nib << (4 * w4_slot(e));
        }
        dst[d] = w;
    }
}

void w4_gpu_to_logical(const uint32_t* src, int64_t cols, uint8_t* dst) {
    memset(dst, 0, (size_t)(cols / 2));
    for (int64_t d = 0; d < cols / 8; ++d)
        for (int e = 0; e < 8; ++e) {
            const int64_t k = d * 8 + e;
            const uint8_t nib = (uint8_t)((src[d] >> (4 * w4_slot(e))) & 15);
            dst[k >> 1] |= (k & 1) ? (uint8_t)(nib << 4) : nib;
        }
}

struct MatRef {
    uint32_t* w4 = nullptr;
    int8_t* i8 = nullptr;
    uint16_t* scales = nullptr;
    int64_t rows = 0, cols = 0;
    int64_t row_stride = 1;   // GPU rows between consecutive logical rows (2 for gate/up)
};

int mat_ref(aw4_model* m, int layer, int kind, MatRef* r) {
    const aw4_config* c = &m->cfg;
    if (kind == AW4_T_LM_HEAD) {
        if (layer != -1 || c->vocab <= 0) return fail(m, AW4_E_INVAL, "lm_head needs layer -1 and vocab > 0");
        r->i8 = m->lm_codes;
        r->scales = m->lm_scales;
        r->rows = c->vocab;
        r->cols = c->hidden;
        return AW4_OK;
    }
    const int64_t H = c->hidden, F = c->ffn;
    const bool draft_layer = c->draft_vocab > 0 && layer == c->n_layers;
    if (kind == AW4_T_DRAFT_FUSE) {
        if (!draft_layer) return fail(m, AW4_E_INVAL, "the draft fuse matrix sits at layer n_layers of a draft model");
        *r = {m->w_fuse, nullptr, m->s_fuse, H, 2 * H, 1};
        return AW4_OK;
    }
    if (kind < 0 || kind > 4 || layer < 0 || (layer >= c->n_layers && !draft_layer))
        return fail(m, AW4_E_INVAL, "bad layer/kind");
    LayerBufs& b = draft_layer ? m->D : m->L[layer];
    switch (kind) {
        case AW4_T_MIX_IN: *r = {b.w_in, nullptr, b.s_in, b.in_rows, H, 1}; break;
        case AW4_T_MIX_OUT: *r = {b.w_out, nullptr, b.s_out, H, b.out_cols, 1}; break;
        case AW4_T_FFN_GATE: *r = {b.w_gu, nullptr, b.s_gu, F, H, 2}; break;
        case AW4_T_FFN_UP: *r = {b.w_gu + H / 8, nullptr, b.s_gu + H / 32, F, H, 2}; break;
        case AW4_T_FFN_DOWN: *r = {b.w_down, nullptr, b.s_down, H, F, 1}; break;
    }
    return AW4_OK;
}

// rows x cols of tensor (layer, kind) of config c (vectors: 1 x n); false
// when the config has no such tensor.  Layer -1 holds the global tensors,
// layer n_layers the draft head's (draft_vocab > 0).
bool cfg_tensor_shape(const aw4_config* c, int layer, int kind, int64_t* rows, int64_t* cols) {
    const int64_t H = c->hidden, F = c->ffn;
    const bool dl = c->draft_vocab > 0 && layer == c->n_layers;
    const bool ll = layer >= 0 && layer < c->n_layers;
    const char t = ll ? c->layer_pattern[layer] : dl ? 'A' : 0;
    const bool glob = layer == -1;
    int64_t r = -1, k = -1;
    switch (kind) {
        case AW4_T_MIX_IN: if (t) { r = mix_in_rows(c, t); k = H; } break;
        case AW4_T_MIX_OUT: if (t) { r = H; k = mix_out_cols(c, t); } break;
        case AW4_T_FFN_GATE:
        case AW4_T_FFN_UP: if (t) { r = F; k = H; } break;
        case AW4_T_FFN_DOWN: if (t) { r = H; k = F; } break;
        case AW4_T_LM_HEAD: if (glob && c->vocab > 0) { r = c->vocab; k = H; } break;
        case AW4_T_NORM_MIX:
        case AW4_T_NORM_FFN: if (t) { r = 1; k = H; } break;
        case AW4_T_NORM_GATED: if (ll && t == 'G') { r = 1; k = c->gdn_head_dim; } break;
        case AW4_T_A_BIAS: if (ll && t == 'G') { r = 1; k = c->gdn_v_heads; } break;
        case AW4_T_NORM_FINAL: if (glob && c->vocab > 0) { r = 1; k = H; } break;
        case AW4_T_RHT_SIGNS:
            if (glob && (strchr(c->layer_pattern, 'A') || c->draft_vocab > 0)) { r = 1; k = c->attn_head_dim; }
            break;
        case AW4_T_DRAFT_FUSE: if (dl) { r = H; k = 2 * H; } break;
        case AW4_T_DRAFT_NORM_EMB:
        case AW4_T_DRAFT_NORM_HID:
        case AW4_T_DRAFT_NORM_OUT: if (dl) { r = 1; k = H; } break;
        case AW4_T_DRAFT_MAP: if (dl) { r = 1; k = c->draft_vocab; } break;
        default: break;
    }
    if (r < 0) return false;
    *rows = r;
    *cols = k;
    return true;
}

bool is_matrix_kind(int kind) { return (kind >= AW4_T_MIX_IN && kind <= AW4_T_LM_HEAD) || kind == AW4_T_DRAFT_FUSE; }

// every tensor of the config, none of it set yet
std::vector<TensorSlot> all_slots(const aw4_config* c) {
    std::vector<TensorSlot> v;
    for (int layer = -1; layer <= c->n_layers; ++layer)
        for (int kind = AW4_T_MIX_IN; kind <= AW4_T_DRAFT_MAP; ++kind) {
            int64_t r, k;
            if (!cfg_tensor_shape(c, layer, kind, &r, &k)) continue;
            TensorSlot t;
            t.layer = layer;
            t.kind = kind;
            t.rows = r;
            t.done.assign((size_t)r, false);
            v.push_back(std::move(t));
        }
    return v;
}

// rows [r0, r0 + n) of tensor (layer, kind) now hold values
void mark_rows(aw4_model* m, int layer, int kind, int64_t r0, int64_t n) {
    for (TensorSlot& t : m->slots) {
        if (t.layer != layer || t.kind != kind) continue;
        const bool was = t.ndone == t.rows;
        for (int64_t r = r0; r < r0 + n && r < t.rows; ++r)
            if (!t.done[(size_t)r]) {
                t.done[(size_t)r] = true;
                ++t.ndone;
            }
        if (!was && t.ndone == t.rows) --m->slots_missing;
        return;
    }
}

// AW4_E_STATE until every tensor of the config has been given values
int need_weights(aw4_model* m) {
    if (m->slots_missing == 0) return AW4_OK;
    for (const TensorSlot& t : m->slots)
        if (t.ndone < t.rows)
            return fail(m, AW4_E_STATE, "weights not loaded: tensor (layer " + std::to_string(t.layer) + ", kind " +
                                            std::to_string(t.kind) + ") has " + std::to_string(t.rows - t.ndone) +
                                            " of " + std::to_string(t.rows) + " rows unset");
    return AW4_OK;
}

// a decode call with a recent window needs rings that hold no position after
// the current one; the call then writes the rings itself
int need_fresh_window(aw4_model* m) {
    for (bool f : m->win_fresh)
        if (!f)
            return fail(m, AW4_E_STATE, "the position moved back: import every attention layer's recent-window "
                                        "ring (aw4_import_state_win) before decoding");
    m->win_imported.assign(m->win_imported.size(), false);
    return AW4_OK;
}

// ---------------------------------------------------------------- weight blob
// Layout (little-endian): "AW4W", uint32 version 4, the shape fields of the
// config as int32 (hidden, ffn, vocab, n_layers, gdn_qk_heads, gdn_v_heads,
// gdn_head_dim, attn_q_heads, attn_kv_heads, attn_head_dim, group,
// draft_vocab), layer_pattern as 128 bytes (NUL padded), uint32 tensor count,
// then per tensor int32 layer, int32 kind, int64 rows, int64 cols, uint64
// payload bytes and the payload: matrices their logical codes then fp16 scale
// bits, vectors n fp32 values, the draft map n int32 ids.
constexpr uint32_t kBlobVersion = 4;
constexpr int kBlobShapeFields = 12;
constexpr uint64_t kBlobHeader = 4 + 4 + 4 * kBlobShapeFields + 128 + 4;

struct BlobTensor {
    int32_t layer, kind;
    int64_t rows, cols;
    const uint8_t* payload;
};

void blob_shape_fields(const aw4_config* c, int32_t* f) {
    const int32_t v[kBlobShapeFields] = {c->hidden, c->ffn, c->vocab, c->n_layers, c->gdn_qk_heads, c->gdn_v_heads,
                                         c->gdn_head_dim, c->attn_q_heads, c->attn_kv_heads, c->attn_head_dim,
                                         c->group, c->draft_vocab};
    memcpy(f, v, sizeof(v));
}

bool f16_bits_ok(uint16_t b) { return (b & 0x8000u) == 0 && (b & 0x7C00u) != 0x7C00u; }   // finite, not negative

// Checks a blob against config c (pure host: nothing is read beyond
// [p, p + bytes) and nothing is enqueued).  With apply set, calls it for every
// tensor of a blob already checked.  AW4_E_FORMAT with *why on the first fault.
template <class F>
int walk_blob(const aw4_config* c, const uint8_t* p, uint64_t bytes, std::string* why, F&& apply) {
    auto bad = [&](const std::string& w) {
        *why = w;
        return AW4_E_FORMAT;
    };
    const uint8_t* end = p + bytes;
    auto left = [&]() { return (uint64_t)(end - p); };
    if (bytes < kBlobHeader) return bad("blob shorter than its header");
    if (memcmp(p, "AW4W", 4) != 0) return bad("bad magic");
    uint32_t ver;
    memcpy(&ver, p + 4, 4);
    if (ver != kBlobVersion) return bad("unsupported blob version " + std::to_string(ver));
    int32_t f[kBlobShapeFields], want[kBlobShapeFields];
    memcpy(f, p + 8, sizeof(f));
    blob_shape_fields(c, want);
    static const char* names[kBlobShapeFields] = {"hidden", "ffn", "vocab", "n_layers", "gdn_qk_heads",
                                                   "gdn_v_heads", "gdn_head_dim", "attn_q_heads", "attn_kv_heads",
                                                   "attn_head_dim", "group", "draft_vocab"};
    for (int i = 0; i < kBlobShapeFields; ++i)
        if (f[i] != want[i])
            return bad(std::string("blob was made for another config: ") + names[i] + " " + std::to_string(f[i]) +
                       " != " + std::to_string(want[i]));
    char pat[129] = {0};
    memcpy(pat, p + 8 + 4 * kBlobShapeFields, 128);
    if (strncmp(pat, c->layer_pattern, 128) != 0) return bad("blob was made for another config: layer_pattern");
    uint32_t count;
    memcpy(&count, p + kBlobHeader - 4, 4);
    p += kBlobHeader;
    std::vector<std::pair<int, int>> seen;
    for (uint32_t t = 0; t < count; ++t) {
        if (left() < 32) return bad("truncated tensor header " + std::to_string(t));
        BlobTensor bt;
        uint64_t nb;
        memcpy(&bt.layer, p, 4);
        memcpy(&bt.kind, p + 4, 4);
        memcpy(&bt.rows, p + 8, 8);
        memcpy(&bt.cols, p + 16, 8);
        memcpy(&nb, p + 24, 8);
        p += 32;
        const std::string tn = "tensor (layer " + std::to_string(bt.layer) + ", kind " + std::to_string(bt.kind) + ")";
        int64_t er = 0, ec = 0;
        if (!cfg_tensor_shape(c, bt.layer, bt.kind, &er, &ec)) return bad(tn + " is not part of the config");
        if (er != bt.rows || ec != bt.cols) return bad(tn + " has the wrong shape");
        for (auto& s2 : seen)
            if (s2.first == bt.layer && s2.second == bt.kind) return bad(tn + " appears twice");
        seen.emplace_back(bt.layer, bt.kind);
        uint64_t want_nb;
        if (is_matrix_kind(bt.kind))
            want_nb = (uint64_t)bt.rows * bt.cols / (bt.kind == AW4_T_LM_HEAD ? 1 : 2) + (uint64_t)bt.rows * (bt.cols / 32) * 2;
        else
            want_nb = (uint64_t)bt.cols * 4;
        if (nb != want_nb) return bad(tn + " payload size mismatch");
        if (left() < nb) return bad(tn + " payload truncated");
        bt.payload = p;
        constexpr bool kCheck = std::is_same_v<std::decay_t<F>, std::nullptr_t>;
        if constexpr (kCheck) {
            // value checks: codes inside the codec's range, scales finite and
            // not negative, signs +-1, finite vectors, a valid map
            if (is_matrix_kind(bt.kind)) {
                const uint64_t cb = nb - (uint64_t)bt.rows * (bt.cols / 32) * 2;
                if (bt.kind == AW4_T_LM_HEAD) {
                    for (uint64_t i = 0; i < cb; ++i)
                        if (p[i] == 0x80) return bad(tn + " holds int8 code -128 (outside -127..127)");
                } else {
                    for (uint64_t i = 0; i < cb; ++i)
                        if ((p[i] & 15) == 0 || (p[i] >> 4) == 0) return bad(tn + " holds W4 code -8 (outside -7..7)");
                }
                for (uint64_t i = cb; i < nb; i += 2) {
                    uint16_t b;
                    memcpy(&b, p + i, 2);
                    if (!f16_bits_ok(b)) return bad(tn + " holds a negative or non-finite scale");
                }
            } else if (bt.kind == AW4_T_DRAFT_MAP) {
                std::vector<int32_t> ids((size_t)bt.cols);
                memcpy(ids.data(), p, (size_t)nb);
                std::sort(ids.begin(), ids.end());
                for (size_t i = 0; i < ids.size(); ++i)
                    if (ids[i] < 0 || ids[i] >= c->vocab || (i && ids[i] == ids[i - 1]))
                        return bad(tn + " ids must be distinct and in [0, vocab)");
            } else {
                for (int64_t i = 0; i < bt.cols; ++i) {
                    float v;
                    memcpy(&v, p + 4 * i, 4);
                    if (!std::isfinite(v)) return bad(tn + " holds a non-finite value");
                    if (bt.kind == AW4_T_RHT_SIGNS && v != 1.0f && v != -1.0f) return bad(tn + " signs must be +-1");
                }
            }
        } else {
            const int rc = apply(bt);
            if (rc) return rc;
        }
        p += nb;
    }
    if (p != end) return bad("trailing bytes after the last tensor");
    return AW4_OK;
}

// ---------------------------------------------------------------- static scratch
// For callers that cannot allocate (code under graph capture, serving loops,
// harnesses that forbid hipMalloc): aw4_decode_step_static keeps the decode
// step's split partials and head partials in this file-scope device array
// instead of the arena.  Each device holds its own copy until the process
// ends; its address comes from hipGetSymbolAddress, once per device, at
// aw4_create with that device current (the array's name is not a device
// address in host code).  Every call on a device shares that device's copy.
constexpr uint64_t kStaticScratchBytes = 4ull << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_dev[kMaxDevices] = {};

// the current device's copy of the array (resolved on first use per device)
hipError_t static_scratch_of(int dev, uint8_t** out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_dev[dev] = (uint8_t*)ptr;
    }
    *out = g_scratch_dev[dev];
    return hipSuccess;
}

// bytes of static scratch the single-token step needs: one token's rows of
// attention partials ([nq][splits][d] then [nq][splits][2]) and the head's
// per-block best value and index
uint64_t static_step_bytes(const aw4_model* m) {
    const aw4_config* c = &m->cfg;
    const bool attn = strchr(c->layer_pattern, 'A') != nullptr;
    uint64_t part = attn ? (uint64_t)c->attn_q_heads * (m->nsplit + m->nsplit_w) * (c->attn_head_dim + 2) * 4 : 0;
    part = (part + 255) & ~uint64_t(255);
    const uint64_t head = (uint64_t)m->nhead_blocks * 4;
    return part + 2 * ((head + 255) & ~uint64_t(255));
}

// ---------------------------------------------------------------- step sequence
// One pre-norm block on the single residual x: mixer input projection, the
// mixer (GDN step, or attention over the cache of committed length *posp with
// the token appended at *posp + pos_offset), its output projection and the FFN,
// both added to x.
int enqueue_block(aw4_model* m, LayerBufs& b, float* x, const int32_t* posp, int pos_offset) {
    const aw4_config* c = &m->cfg;
    hipStream_t s = m->stream;
    const int H = c->hidden, F = c->ffn;
    {
        GemvArgs gi{};
        gi.codes = b.w_in;
        gi.scales = b.s_in;
        gi.rows = (int)b.in_rows;
        gi.K = H;
        gi.x = x;
        gi.nw = b.norm_mix;
        gi.eps = c->rms_eps;
        gi.y = m->proj;
        HIPCHK(m, launch_gemv(PRO_NORM, EPI_STORE, gi, s));
    }
    {
        if (b.type == 'G') {
            GdnArgs ga{m->proj, b.a_bias, b.S, m->obuf, c->gdn_qk_heads, c->gdn_v_heads, c->gdn_head_dim, c->rms_eps};
            HIPCHK(m, launch_gdn(ga, s));
            GemvArgs go{};
            go.codes = b.w_out;
            go.scales = b.s_out;
            go.rows = H;
            go.K = (int)b.out_cols;
            go.x = m->obuf;
            go.nw = b.norm_gated;
            go.z = m->proj + 2LL * c->gdn_qk_heads * c->gdn_head_dim + (int64_t)c->gdn_v_heads * c->gdn_head_dim;
            go.gated_d = c->gdn_head_dim;
            go.eps = c->rms_eps;
            go.y = x;
            HIPCHK(m, launch_gemv(PRO_GATED, EPI_RESID, go, s));
        } else {
            AttnArgs aa{};
            aa.pos_offset = pos_offset;
            aa.nt = 1;
            aa.append = 1;
            aa.proj = m->proj;
            aa.kc = b.kc;
            aa.ks = b.ks;
            aa.vc = b.vc;
            aa.vs = b.vs;
            aa.signs = m->signs;
            aa.pos = posp;
            aa.part = m->step_part;
            aa.prow = m->step_prow;
            aa.max_ctx = c->max_ctx;
            aa.nq = c->attn_q_heads;
            aa.nkv = c->attn_kv_heads;
            aa.d = c->attn_head_dim;
            aa.nsplit = m->nsplit;
            aa.fmt = c->kv_format;
            if (b.kw) {
                // recent window: the sweep before the window, then the
                // window's sweep, which appends the token (codes and fp16
                // ring entry) first
                aa.win = c->kv_window;
                aa.nsplit_w = m->nsplit_w;
                aa.kw = b.kw;
                aa.vw = b.vw;
                aa.append = 0;
                HIPCHK(m, launch_attn(aa, s));
                aa.append = 1;
                HIPCHK(m, launch_attn_win(aa, s));
            } else {
                HIPCHK(m, launch_attn(aa, s));
            }
            CombineArgs ca{pos_offset, 1, 0, m->step_part, m->proj, m->signs, posp, m->abuf, aa.prow, c->attn_q_heads,
                           c->attn_kv_heads, c->attn_head_dim, m->nsplit, 0, aa.win, aa.nsplit_w, c->kv_format};
            HIPCHK(m, launch_combine(ca, s));
            GemvArgs go{};
            go.codes = b.w_out;
            go.scales = b.s_out;
            go.rows = H;
            go.K = (int)b.out_cols;
            go.h = m->abuf;
            go.y = x;
            HIPCHK(m, launch_gemv(PRO_LOADH, EPI_RESID, go, s));
        }
        GemvArgs gf{};
        gf.codes = b.w_gu;
        gf.scales = b.s_gu;
        gf.rows = 2 * F;
        gf.K = H;
        gf.x = x;
        gf.nw = b.norm_ffn;
        gf.eps = c->rms_eps;
        gf.hout = m->hbuf;
        HIPCHK(m, launch_gemv(PRO_NORM, EPI_SWIGLU, gf, s));
        GemvArgs gd{};
        gd.codes = b.w_down;
        gd.scales = b.s_down;
        gd.rows = H;
        gd.K = F;
        gd.h = m->hbuf;
        gd.y = x;
        HIPCHK(m, launch_gemv(PRO_LOADH, EPI_RESID, gd, s));
    }
    return AW4_OK;
}

int enqueue_layers(aw4_model* m) {
    for (int l = 0; l < m->cfg.n_layers; ++l) {
        int rc = enqueue_block(m, m->L[l], m->x, &m->ctl->pos, 0);
        if (rc) return rc;
    }
    return AW4_OK;
}

// one launch of a phase for layer l (timing); returns its algorithmic bytes
int enqueue_phase(aw4_model* m, int phase, int l, uint64_t* bytes) {
    const aw4_config* c = &m->cfg;
    hipStream_t s = m->stream;
    const int H = c->hidden, F = c->ffn;
    LayerBufs& b = m->L[l];
    auto w4b = [](int64_t rows, int64_t cols) { return (uint64_t)(rows * cols / 2 + rows * (cols / 32) * 2); };
    GemvArgs g{};
    g.eps = c->rms_eps;
    switch (phase) {
        case AW4_PHASE_FFN_GATE_UP:
            g.codes = b.w_gu; g.scales = b.s_gu; g.rows = 2 * F; g.K = H; g.x = m->x; g.nw = b.norm_ffn;
            g.hout = m->hbuf;
            *bytes = w4b(2LL * F, H) + (uint64_t)H * 8 + (uint64_t)F * 2;
            HIPCHK(m, launch_gemv(PRO_NORM, EPI_SWIGLU, g, s));
            break;
        case AW4_PHASE_FFN_DOWN:
            g.codes = b.w_down; g.scales = b.s_down; g.rows = H; g.K = F; g.h = m->hbuf; g.y = m->x;
            *bytes = w4b(H, F) + (uint64_t)F * 2 + (uint64_t)H * 8;
            HIPCHK(m, launch_gemv(PRO_LOADH, EPI_RESID, g, s));
            break;
        case AW4_PHASE_MIX_IN:
            g.codes = b.w_in; g.scales = b.s_in; g.rows = (int)b.in_rows; g.K = H; g.x = m->x; g.nw = b.norm_mix;
            g.y = m->proj;
            *bytes = w4b(b.in_rows, H) + (uint64_t)H * 8 + (uint64_t)b.in_rows * 4;
            HIPCHK(m, launch_gemv(PRO_NORM, EPI_STORE, g, s));
            break;
        case AW4_PHASE_HEAD:
        case AW4_PHASE_DRAFT_HEAD: {
            // int8 rows (+ fp16 scales) of the full table or of the mapped ids, the
            // normalised input, one fp32 score per row
            const bool mapped = phase == AW4_PHASE_DRAFT_HEAD;
            if (c->vocab <= 0 || (mapped && (c->draft_vocab <= 0 || !m->map_set)))
                return fail(m, AW4_E_STATE, "no such head");
            const int rows = mapped ? c->draft_vocab : c->vocab;
            HeadArgs ha{m->lm_codes, m->lm_scales, mapped ? m->dmap : nullptr, rows, H, m->x,
                        mapped ? m->dn_out : m->norm_final, c->rms_eps, mapped ? m->dscore : m->logits,
                        mapped ? m->dpv : m->pv, mapped ? m->dpi : m->pi};
            *bytes = (uint64_t)rows * (H + H / 16) + (uint64_t)H * 8 + (uint64_t)rows * (mapped ? 8 : 4);
            HIPCHK(m, launch_head(ha, s));
            break;
        }
        case AW4_PHASE_PREFILL_GATE_UP: {
            // the prefill chunk's gate/up GEMM with SwiGLU: 2 M N K flops
            const int M = m->pchunk_max;
            if (M <= 0) return fail(m, AW4_E_STATE, "no chunked prefill for this shape");
            *bytes = 2ULL * M * (2ULL * F) * H;
            GemmArgs ga{b.w_gu, b.s_gu, 2 * F, H, M, m->pa, m->pa_ld, nullptr, 0, m->pf, F,
                        m->gpart, kGemmSplitSlots, 0, 0};
            HIPCHK(m, launch_gemm_w4(EPI_SWIGLU, ga, s));
            break;
        }
        default:
            return fail(m, AW4_E_INVAL, "unknown phase");
    }
    return AW4_OK;
}

// Gated attention of M tokens at cache positions *posp .. *posp + M - 1 (their
// projections at proj, rows in_rows apart): all M tokens' K and V are appended
// first, then one launch of sweeps of up to tps tokens each (grid z) reads the
// cache (each token masked to its own position) and one combine merges all M;
// the o-projection adds into the M residuals at x.
int enqueue_attn_multi(aw4_model* m, LayerBufs& b, int M, float* x, float* proj, const int32_t* posp) {
    const aw4_config* c = &m->cfg;
    hipStream_t s = m->stream;
    const int H = c->hidden;
    const int64_t od = (int64_t)c->attn_q_heads * c->attn_head_dim;
    AttnArgs aa{};
    aa.nt = M;
    aa.sproj = b.in_rows;
    aa.proj = proj;
    aa.kc = b.kc; aa.ks = b.ks; aa.vc = b.vc; aa.vs = b.vs;
    aa.signs = m->signs; aa.pos = posp; aa.part = m->part; aa.prow = kSweepRows * c->attn_q_heads;
    aa.max_ctx = c->max_ctx; aa.nq = c->attn_q_heads; aa.nkv = c->attn_kv_heads;
    aa.d = c->attn_head_dim; aa.nsplit = m->nsplit;
    HIPCHK(m, launch_append(aa, s));
    aa.zfast = M > attn_tokens_per_sweep(c->attn_head_dim, c->attn_q_heads, c->attn_kv_heads) ? 1 : 0;
    HIPCHK(m, launch_attn(aa, s));
    CombineArgs ca{0, M, b.in_rows, m->part, proj, m->signs, posp, m->va, aa.prow,
                   c->attn_q_heads, c->attn_kv_heads, c->attn_head_dim, m->nsplit};
    HIPCHK(m, launch_combine(ca, s));
    GemvMultiArgs go{};
    go.codes = b.w_out; go.scales = b.s_out; go.rows = H; go.K = (int)b.out_cols; go.M = M;
    go.h = m->va; go.sh = od; go.y = x; go.sy = H;
    HIPCHK(m, launch_gemv_multi(PRO_LOADH, EPI_RESID, go, s));
    return AW4_OK;
}

// FFN of M residuals at x (rows H apart), added into them
int enqueue_ffn_multi(aw4_model* m, LayerBufs& b, int M, float* x) {
    const aw4_config* c = &m->cfg;
    hipStream_t s = m->stream;
    const int H = c->hidden, F = c->ffn;
    GemvMultiArgs gf{};
    gf.codes = b.w_gu; gf.scales = b.s_gu; gf.rows = 2 * F; gf.K = H; gf.M = M;
    gf.x = x; gf.sx = H; gf.nw = b.norm_ffn; gf.eps = c->rms_eps; gf.hout = m->vh; gf.so = m->hlen;
    HIPCHK(m, launch_gemv_multi(PRO_NORM, EPI_SWIGLU, gf, s));
    GemvMultiArgs gd{};
    gd.codes = b.w_down; gd.scales = b.s_down; gd.rows = H; gd.K = F; gd.M = M;
    gd.h = m->vh; gd.sh = m->hlen; gd.y = x; gd.sy = H;
    HIPCHK(m, launch_gemv_multi(PRO_LOADH, EPI_RESID, gd, s));
    return AW4_OK;
}

// The verify pass: M tokens (ctl->vtok) at positions pos .. pos+M-1 through
// every layer with one sweep over the weights, the head over the M residuals,
// acceptance, then the commit (GDN replay of the accepted prefix, pos advance).
int enqueue_verify(aw4_model* m, int M, int k, const float* dev_q, float temperature) {
    const aw4_config* c = &m->cfg;
    hipStream_t s = m->stream;
    const int H = c->hidden;
    HIPCHK(m, launch_embed_multi(m->lm_codes, m->lm_scales, H, m->ctl, M, m->vx, s));
    int gi_layer = 0;
    for (int l = 0; l < c->n_layers; ++l) {
        LayerBufs& b = m->L[l];
        float* proj = b.type == 'G' ? m->vproj_g[gi_layer] : m->vproj_a;
        GemvMultiArgs gi{};
        gi.codes = b.w_in; gi.scales = b.s_in; gi.rows = (int)b.in_rows; gi.K = H; gi.M = M;
        gi.x = m->vx; gi.sx = H; gi.nw = b.norm_mix; gi.eps = c->rms_eps; gi.y = proj; gi.sy = b.in_rows;
        HIPCHK(m, launch_gemv_multi(PRO_NORM, EPI_STORE, gi, s));
        if (b.type == 'G') {
            GdnMultiArgs ga{};
            ga.proj = proj; ga.sproj = b.in_rows; ga.a_bias = b.a_bias; ga.S = b.S; ga.o = m->vo;
            ga.so = (int64_t)c->gdn_v_heads * c->gdn_head_dim; ga.nqk = c->gdn_qk_heads; ga.nv = c->gdn_v_heads;
            ga.d = c->gdn_head_dim; ga.M = M; ga.eps = c->rms_eps; ga.replay = 0; ga.commit_n = nullptr;
            HIPCHK(m, launch_gdn_multi(ga, s));
            GemvMultiArgs go{};
            go.codes = b.w_out; go.scales = b.s_out; go.rows = H; go.K = (int)b.out_cols; go.M = M;
            go.x = m->vo; go.sx = ga.so; go.nw = b.norm_gated;
            go.z = proj + 2LL * c->gdn_qk_heads * c->gdn_head_dim + (int64_t)c->gdn_v_heads * c->gdn_head_dim;
            go.sz = b.in_rows; go.gated_d = c->gdn_head_dim; go.eps = c->rms_eps; go.y = m->vx; go.sy = H;
            HIPCHK(m, launch_gemv_multi(PRO_GATED, EPI_RESID, go, s));
            ++gi_layer;
        } else {
            int rc = enqueue_attn_multi(m, b, M, m->vx, proj, &m->ctl->pos);
            if (rc) return rc;
        }
        int rc = enqueue_ffn_multi(m, b, M, m->vx);
        if (rc) return rc;
    }
    HeadMultiArgs ha{m->lm_codes, m->lm_scales, c->vocab, c->hidden, M, m->vx, m->norm_final, c->rms_eps,
                     m->vlogits, m->vpv, m->vpi};
    HIPCHK(m, launch_head_multi(ha, s));
    AcceptArgs ac{};
    ac.ctl = m->ctl; ac.logits = m->vlogits; ac.q = dev_q; ac.V = c->vocab; ac.k = k;
    ac.greedy = temperature == 0.f; ac.inv_t = temperature == 0.f ? 1.f : 1.f / temperature;
    ac.zpart = m->vzpart; ac.wpart = m->vwpart;
    HIPCHK(m, launch_accept(ac, m->vpv, m->vpi, m->nhead_blocks, s));
    // commit: replay the accepted prefix into the GDN states (every layer's in
    // one launch, up to kMaxReplayLayers at a time), advance the position
    GdnReplayArgs rp{};
    gi_layer = 0;
    for (int l = 0; l < c->n_layers; ++l) {
        LayerBufs& b = m->L[l];
        if (b.type != 'G') continue;
        if (rp.nlayers == 0) {
            GdnMultiArgs& ga = rp.a;
            ga.sproj = b.in_rows; ga.o = nullptr; ga.so = 0; ga.nqk = c->gdn_qk_heads; ga.nv = c->gdn_v_heads;
            ga.d = c->gdn_head_dim; ga.M = M; ga.eps = c->rms_eps; ga.replay = 1; ga.commit_n = &m->ctl->vcommit;
        }
        rp.proj[rp.nlayers] = m->vproj_g[gi_layer++];
        rp.a_bias[rp.nlayers] = b.a_bias;
        rp.S[rp.nlayers] = b.S;
        if (++rp.nlayers == kMaxReplayLayers) {
            HIPCHK(m, launch_gdn_replay(rp, s));
            rp.nlayers = 0;
        }
    }
    if (rp.nlayers > 0) HIPCHK(m, launch_gdn_replay(rp, s));
    HIPCHK(m, launch_commit_pos(m->ctl, s));
    return AW4_OK;
}

// embed ctl->token, run the layers, then either the head (argmax -> ctl->token,
// pos += 1) or just pos += 1
int enqueue_step(aw4_model* m, bool head) {
    const aw4_config* c = &m->cfg;
    hipStream_t s = m->stream;
    HIPCHK(m, launch_embed(m->lm_codes, m->lm_scales, c->hidden, m->ctl, m->x, s));
    int rc = enqueue_layers(m);
    if (rc) return rc;
    if (head) {
        HeadArgs ha{m->lm_codes, m->lm_scales, nullptr, c->vocab, c->hidden, m->x, m->norm_final, c->rms_eps,
                    m->logits, m->step_pv, m->step_pi};
        HIPCHK(m, launch_head(ha, s));
        HIPCHK(m, launch_head_final(m->step_pv, m->step_pi, m->nhead_blocks, m->ctl, m->ring, m->ring_cap, s));
    } else {
        HIPCHK(m, launch_advance(m->ctl, s));
    }
    return AW4_OK;
}

// The draft head's block on M entries (page 5, bs178.com llamAmpere article,
// point 四; block structure a reading): input from token tok[i] (device) and
// hidden hin + i sh, the fuse projection into xd rows 0..M-1, then its
// gated-attention block over its own cache, the entries written at
// ctl->dpos + pos_offset + i.
int enqueue_draft_block(aw4_model* m, int M, const int32_t* tok, const float* hin, int64_t sh, int pos_offset) {
    const aw4_config* c = &m->cfg;
    hipStream_t s = m->stream;
    const int H = c->hidden;
    DraftEmbedArgs de{m->lm_codes, m->lm_scales, tok, hin, sh, m->dn_emb, m->dn_hid, m->ubuf, H, M, c->rms_eps};
    HIPCHK(m, launch_draft_embed(de, s));
    if (M == 1) {
        GemvArgs gf{};
        gf.codes = m->w_fuse; gf.scales = m->s_fuse; gf.rows = H; gf.K = 2 * H; gf.h = m->ubuf; gf.y = m->xd;
        HIPCHK(m, launch_gemv(PRO_LOADH, EPI_STORE, gf, s));
        return enqueue_block(m, m->D, m->xd, &m->ctl->dpos, pos_offset);
    }
    if (pos_offset != 0) return fail(m, AW4_E_INVAL, "multi-entry draft steps start at the committed length");
    LayerBufs& b = m->D;
    GemvMultiArgs gf{};
    gf.codes = m->w_fuse; gf.scales = m->s_fuse; gf.rows = H; gf.K = 2 * H; gf.M = M;
    gf.h = m->ubuf; gf.sh = 2 * H; gf.y = m->xd; gf.sy = H;
    HIPCHK(m, launch_gemv_multi(PRO_LOADH, EPI_STORE, gf, s));
    GemvMultiArgs gi{};
    gi.codes = b.w_in; gi.scales = b.s_in; gi.rows = (int)b.in_rows; gi.K = H; gi.M = M;
    gi.x = m->xd; gi.sx = H; gi.nw = b.norm_mix; gi.eps = c->rms_eps; gi.y = m->vproj_a; gi.sy = b.in_rows;
    HIPCHK(m, launch_gemv_multi(PRO_NORM, EPI_STORE, gi, s));
    int rc = enqueue_attn_multi(m, b, M, m->xd, m->vproj_a, &m->ctl->dpos);
    if (rc) return rc;
    return enqueue_ffn_multi(m, b, M, m->xd);
}

// Mapped scores of xd row `row` (the draft output norm, then the int8 table
// rows of the map) and the choice of draft j; commit entries are added to the
// draft cache length once the step's cache reads are done.
int enqueue_draft_select(aw4_model* m, int row, int j, int commit, float temperature, float* q_row, float* z_row) {
    const aw4_config* c = &m->cfg;
    hipStream_t s = m->stream;
    float* z = z_row ? z_row : m->dscore;
    HeadArgs ha{m->lm_codes, m->lm_scales, m->dmap, c->draft_vocab, c->hidden, m->xd + (int64_t)row * c->hidden,
                m->dn_out, c->rms_eps, z, m->dpv, m->dpi};
    HIPCHK(m, launch_head(ha, s));
    DraftSelArgs ds{};
    ds.ctl = m->ctl; ds.z = z; ds.pv = m->dpv; ds.pi = m->dpi; ds.nb = m->ndhead_blocks;
    ds.map = m->dmap; ds.rmap = m->drmap; ds.Vd = c->draft_vocab; ds.V = c->vocab; ds.j = j; ds.commit = commit;
    ds.greedy = temperature == 0.f; ds.inv_t = temperature == 0.f ? 1.f : 1.f / temperature;
    ds.zpart = m->dzpart; ds.q = q_row;
    HIPCHK(m, launch_draft_select(ds, s));
    return AW4_OK;
}

// ---------------------------------------------------------------- prefill
// W4 GEMM of the chunk: out = x W^T over T tokens
int prefill_gemm(aw4_model* m, int epi, const uint32_t* codes, const uint16_t* scales, int64_t N, int64_t K, int T,
                 const _Float16* x, int64_t ldx, float* y, int64_t ldy, _Float16* hout, int64_t ldo) {
    GemmArgs g{codes, scales, (int32_t)N, (int32_t)K, T, x, ldx, y, ldy, hout, ldo, m->gpart, kGemmSplitSlots,
               0, 0};
    HIPCHK(m, launch_gemm_w4(epi, g, m->stream));
    return AW4_OK;
}

// The layers `layers[0..nl)` on the T residuals x [T][H] of a prefill chunk,
// whose tokens sit at cache positions *posp .. *posp + T - 1: per layer the
// normalised inputs, the mixer input GEMM, the mixer (GDN over the tokens in
// order, or append + causal attention over the cache), the output GEMM into
// x, then the FFN (gate/up GEMM with SwiGLU, down GEMM into x).  Every token
// computes what a decode step computes.
int enqueue_prefill_layers(aw4_model* m, LayerBufs* layers, int nl, int T, float* x, const int32_t* posp) {
    const aw4_config* c = &m->cfg;
    hipStream_t s = m->stream;
    const int64_t H = c->hidden, F = c->ffn;
    const int C = m->pchunk_max;
    int rc;
    for (int l = 0; l < nl; ++l) {
        LayerBufs& b = layers[l];
        HIPCHK(m, launch_norm_rows(x, b.norm_mix, (int)H, c->rms_eps, T, m->pa, m->pa_ld, s));
        if ((rc = prefill_gemm(m, EPI_STORE, b.w_in, b.s_in, b.in_rows, H, T, m->pa, m->pa_ld, m->pp, b.in_rows,
                               nullptr, 0)))
            return rc;
        if (b.type == 'G') {
            const int64_t nvd = (int64_t)c->gdn_v_heads * c->gdn_head_dim;
            GdnPrefillArgs ga{m->pp, b.in_rows, b.a_bias, b.S, m->pqn, m->pkn, m->pab, m->po, nvd,
                              c->gdn_qk_heads, c->gdn_v_heads, c->gdn_head_dim, T, c->rms_eps};
            HIPCHK(m, launch_gdn_prefill(ga, b.norm_gated, m->pa, nvd, s));
            if ((rc = prefill_gemm(m, EPI_RESID, b.w_out, b.s_out, H, nvd, T, m->pa, nvd, x, H, nullptr, 0)))
                return rc;
        } else {
            const int64_t nqd = (int64_t)c->attn_q_heads * c->attn_head_dim;
            AttnArgs aa{};
            aa.nt = T;
            aa.sproj = b.in_rows;
            aa.proj = m->pp;
            aa.kc = b.kc; aa.ks = b.ks; aa.vc = b.vc; aa.vs = b.vs;
            aa.signs = m->signs; aa.pos = posp; aa.part = m->ppart; aa.prow = C * c->attn_q_heads;
            aa.max_ctx = c->max_ctx; aa.nq = c->attn_q_heads; aa.nkv = c->attn_kv_heads;
            aa.d = c->attn_head_dim; aa.nsplit = 1;
            HIPCHK(m, launch_append(aa, s));
            HIPCHK(m, launch_attn(aa, s));
            CombineArgs ca{0, T, b.in_rows, m->ppart, m->pp, m->signs, posp, m->pa, aa.prow, c->attn_q_heads,
                           c->attn_kv_heads, c->attn_head_dim, 1};
            HIPCHK(m, launch_combine(ca, s));
            if ((rc = prefill_gemm(m, EPI_RESID, b.w_out, b.s_out, H, nqd, T, m->pa, nqd, x, H, nullptr, 0)))
                return rc;
        }
        HIPCHK(m, launch_norm_rows(x, b.norm_ffn, (int)H, c->rms_eps, T, m->pa, m->pa_ld, s));
        if ((rc = prefill_gemm(m, EPI_SWIGLU, b.w_gu, b.s_gu, 2 * F, H, T, m->pa, m->pa_ld, nullptr, 0, m->pf, F)))
            return rc;
        if ((rc = prefill_gemm(m, EPI_RESID, b.w_down, b.s_down, H, F, T, m->pf, F, x, H, nullptr, 0))) return rc;
    }
    return AW4_OK;
}

// n prompt tokens in chunks: embedding rows, every layer over the chunk, the
// positions advanced; with a draft head its cache gets the entries of the
// chunk's positions whose next token is known; the last token's hidden state
// ends in x (and through the head in logits when asked).
int enqueue_prefill_chunked(aw4_model* m, const int32_t* tokens, int n, bool want_logits) {
    const aw4_config* c = &m->cfg;
    hipStream_t s = m->stream;
    const int H = c->hidden;
    const bool feed = c->draft_vocab > 0;
    for (int i0 = 0; i0 < n; i0 += m->pchunk) {
        const int T = std::min(m->pchunk, n - i0);
        const bool last = i0 + T == n;
        HIPCHK(m, hipMemcpyAsync(m->ptok, tokens + i0, (size_t)T * 4, hipMemcpyHostToDevice, s));
        HIPCHK(m, launch_embed_rows(m->lm_codes, m->lm_scales, H, m->ptok, T, m->px, s));
        int rc = enqueue_prefill_layers(m, m->L.data(), c->n_layers, T, m->px, &m->ctl->pos);
        if (rc) return rc;
        if (last) HIPCHK(m, launch_copy_f32(m->x, m->px + (int64_t)(T - 1) * H, H, s));
        const int nf = last ? T - 1 : T;
        if (feed && nf > 0) {
            // draft head entries: (hidden of position i0 + t, token i0 + t + 1)
            HIPCHK(m, hipMemcpyAsync(m->pnext, tokens + i0 + 1, (size_t)nf * 4, hipMemcpyHostToDevice, s));
            DraftEmbedArgs de{m->lm_codes, m->lm_scales, m->pnext, m->px, H, m->dn_emb, m->dn_hid, m->pa, H, nf,
                              c->rms_eps};
            HIPCHK(m, launch_draft_embed(de, s));
            if ((rc = prefill_gemm(m, EPI_STORE, m->w_fuse, m->s_fuse, H, 2LL * H, nf, m->pa, 2LL * H, m->px, H,
                                   nullptr, 0)))
                return rc;
            if ((rc = enqueue_prefill_layers(m, &m->D, 1, nf, m->px, &m->ctl->dpos))) return rc;
            m->host_dpos += nf;
            HIPCHK(m, launch_set_dpos(m->ctl, m->host_dpos, s));
        }
        m->host_pos += T;
        HIPCHK(m, launch_set_ctl(m->ctl, m->host_pos, -1, -1, s));
    }
    if (want_logits) {
        HeadArgs ha{m->lm_codes, m->lm_scales, nullptr, c->vocab, H, m->x, m->norm_final, c->rms_eps, m->logits,
                    m->pv, m->pi};
        HIPCHK(m, launch_head(ha, s));
    }
    return AW4_OK;
}

// One batch step of sequences 0 .. B-1 (tokens and positions already in
// ctl->btok / bpos): the M = B projections, per-sequence GDN steps and
// attention sweeps (grid z), the M = B head and the per-sequence argmax.
int enqueue_batch_step(aw4_model* m, int B) {
    const aw4_config* c = &m->cfg;
    hipStream_t s = m->stream;
    const int H = c->hidden;
    const int64_t sb = (int64_t)m->state_bytes;
    // sequence 0's state pointers (the layers hold the selected sequence's);
    // the kernels add b * state_bytes for sequence b
    const int64_t back = -(int64_t)m->seq * sb;
    auto seq0 = [back](auto* ptr) { return (decltype(ptr))((char*)ptr + back); };
    HIPCHK(m, launch_embed_tokens(m->lm_codes, m->lm_scales, H, m->ctl->btok, B, m->vx, s));
    int gi_layer = 0;
    for (int l = 0; l < c->n_layers; ++l) {
        LayerBufs& b = m->L[l];
        float* proj = b.type == 'G' ? m->vproj_g[gi_layer] : m->vproj_a;
        GemvMultiArgs gi{};
        gi.codes = b.w_in; gi.scales = b.s_in; gi.rows = (int)b.in_rows; gi.K = H; gi.M = B;
        gi.x = m->vx; gi.sx = H; gi.nw = b.norm_mix; gi.eps = c->rms_eps; gi.y = proj; gi.sy = b.in_rows;
        HIPCHK(m, launch_gemv_multi(PRO_NORM, EPI_STORE, gi, s));
        if (b.type == 'G') {
            const int64_t nvd = (int64_t)c->gdn_v_heads * c->gdn_head_dim;
            GdnArgs ga{proj, b.a_bias, seq0(b.S), m->vo, c->gdn_qk_heads, c->gdn_v_heads, c->gdn_head_dim,
                       c->rms_eps, b.in_rows, sb / 4, nvd};
            HIPCHK(m, launch_gdn_batch(ga, B, s));
            GemvMultiArgs go{};
            go.codes = b.w_out; go.scales = b.s_out; go.rows = H; go.K = (int)b.out_cols; go.M = B;
            go.x = m->vo; go.sx = nvd; go.nw = b.norm_gated;
            go.z = proj + 2LL * c->gdn_qk_heads * c->gdn_head_dim + nvd;
            go.sz = b.in_rows; go.gated_d = c->gdn_head_dim; go.eps = c->rms_eps; go.y = m->vx; go.sy = H;
            HIPCHK(m, launch_gemv_multi(PRO_GATED, EPI_RESID, go, s));
            ++gi_layer;
        } else {
            const int64_t od = (int64_t)c->attn_q_heads * c->attn_head_dim;
            AttnArgs aa{};
            aa.nt = B; aa.append = 1; aa.batch = 1; aa.seq_bytes = sb;
            aa.sproj = b.in_rows; aa.proj = proj;
            aa.kc = seq0(b.kc); aa.ks = seq0(b.ks); aa.vc = seq0(b.vc); aa.vs = seq0(b.vs);
            aa.signs = m->signs; aa.pos = m->ctl->bpos; aa.part = m->part; aa.prow = kSweepRows * c->attn_q_heads;
            aa.max_ctx = c->max_ctx; aa.nq = c->attn_q_heads; aa.nkv = c->attn_kv_heads;
            aa.d = c->attn_head_dim; aa.nsplit = m->nsplit;
            HIPCHK(m, launch_attn(aa, s));
            CombineArgs ca{0, B, b.in_rows, m->part, proj, m->signs, m->ctl->bpos, m->va, aa.prow, c->attn_q_heads,
                           c->attn_kv_heads, c->attn_head_dim, m->nsplit, 1};
            HIPCHK(m, launch_combine(ca, s));
            GemvMultiArgs go{};
            go.codes = b.w_out; go.scales = b.s_out; go.rows = H; go.K = (int)b.out_cols; go.M = B;
            go.h = m->va; go.sh = od; go.y = m->vx; go.sy = H;
            HIPCHK(m, launch_gemv_multi(PRO_LOADH, EPI_RESID, go, s));
        }
        int rc = enqueue_ffn_multi(m, b, B, m->vx);
        if (rc) return rc;
    }
    HeadMultiArgs ha{m->lm_codes, m->lm_scales, c->vocab, c->hidden, B, m->vx, m->norm_final, c->rms_eps,
                     m->vlogits, m->vpv, m->vpi};
    HIPCHK(m, launch_head_multi(ha, s));
    HIPCHK(m, launch_head_argmax_multi(m->vpv, m->vpi, m->nhead_blocks, B, m->ctl, s));
    return AW4_OK;
}

int run_step(aw4_model* m, bool head) {
    if (!m->use_graph) return enqueue_step(m, head);
    hipGraphExec_t* ge = head ? &m->g_head : &m->g_nohead;
    if (!*ge) {
        hipGraph_t g = nullptr;
        HIPCHK_RAW(m, hipStreamBeginCapture(m->stream, hipStreamCaptureModeThreadLocal));
        int rc = enqueue_step(m, head);
        hipError_t e = hipStreamEndCapture(m->stream, &g);
        if (rc) {
            if (g) (void)hipGraphDestroy(g);
            return rc;
        }
        if (e != hipSuccess) return fail(m, AW4_E_HIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(e));
        e = hipGraphInstantiate(ge, g, nullptr, nullptr, 0);
        (void)hipGraphDestroy(g);
        if (e != hipSuccess) {
            *ge = nullptr;
            return fail(m, AW4_E_HIP, std::string("hipGraphInstantiate: ") + hipGetErrorString(e));
        }
    }
    HIPCHK(m, hipGraphLaunch(*ge, m->stream));
    return AW4_OK;
}

void drop_graphs(aw4_model* m) {
    if (m->g_head) (void)hipGraphExecDestroy(m->g_head);
    if (m->g_nohead) (void)hipGraphExecDestroy(m->g_nohead);
    m->g_head = m->g_nohead = nullptr;
    for (hipGraphExec_t& g : m->g_batch) {
        if (g) (void)hipGraphExecDestroy(g);
        g = nullptr;
    }
}

int check_model(aw4_model* m) {
    if (!m) return AW4_E_INVAL;
    return AW4_OK;
}

// move every recurrent-state and cache pointer by `delta` sequences
void shift_state(aw4_model* m, int delta) {
    const int64_t d = (int64_t)delta * (int64_t)m->state_bytes;
    auto mv = [d](auto*& ptr) {
        if (ptr) ptr = (std::remove_reference_t<decltype(*ptr)>*)((char*)ptr + d);
    };
    for (LayerBufs& b : m->L) {
        mv(b.S);
        mv(b.kc);
        mv(b.ks);
        mv(b.vc);
        mv(b.vs);
    }
    mv(m->D.kc);
    mv(m->D.ks);
    mv(m->D.vc);
    mv(m->D.vs);
}

// the attention layer whose cache a state call names (n_layers: the draft head's)
LayerBufs* kv_layer(aw4_model* m, int layer) {
    if (!m) return nullptr;
    if (layer >= 0 && layer < m->cfg.n_layers) return m->L[layer].type == 'A' ? &m->L[layer] : nullptr;
    if (layer == m->cfg.n_layers && m->cfg.draft_vocab > 0) return &m->D;
    return nullptr;
}

}  // namespace

// ==================================================================== C ABI
extern "C" {

const char* aw4_status_string(int st) {
    switch (st) {
        case AW4_OK: return "ok";
        case AW4_E_INVAL: return "invalid argument";
        case AW4_E_ARENA: return "arena missing, misaligned or too small";
        case AW4_E_NODEVICE: return "no gfx950 HIP device";
        case AW4_E_HIP: return "HIP runtime error";
        case AW4_E_FORMAT: return "weight blob format error";
        case AW4_E_CTX_FULL: return "context full";
        case AW4_E_TOKEN: return "token out of range";
        case AW4_E_STATE: return "call not valid in the current state";
        default: return "unknown status";
    }
}

const char* aw4_last_error(const aw4_model* m) { return m ? m->err.c_str() : "null model"; }

int aw4_validate_config(const aw4_config* cfg) { return check_config(cfg) ? AW4_E_INVAL : AW4_OK; }

int aw4_workspace_bytes(const aw4_config* cfg, uint64_t* out) {
    if (check_config(cfg) || !out) return AW4_E_INVAL;
    *out = plan_layout(cfg, nullptr, nullptr);
    return AW4_OK;
}

int aw4_create(const aw4_config* cfg, void* dev_arena, uint64_t arena_bytes, void* hip_stream, aw4_model** out) {
    if (!out) return AW4_E_INVAL;
    *out = nullptr;
    if (check_config(cfg)) return AW4_E_INVAL;
    const uint64_t need = plan_layout(cfg, nullptr, nullptr);
    if (!dev_arena || ((uintptr_t)dev_arena & 255) || arena_bytes < need) return AW4_E_ARENA;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return AW4_E_NODEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return AW4_E_NODEVICE;
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return AW4_E_NODEVICE;
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, dev_arena) != hipSuccess || attr.type != hipMemoryTypeDevice)
        return AW4_E_ARENA;
    aw4_model* m = new aw4_model();
    m->cfg = *cfg;
    m->arena = (uint8_t*)dev_arena;
    m->arena_bytes = arena_bytes;
    m->stream = (hipStream_t)hip_stream;
    plan_layout(cfg, m, m->arena);
    m->slots = all_slots(cfg);
    m->slots_missing = (int)m->slots.size();
    m->win_fresh.assign((size_t)cfg->n_layers, true);
    m->win_imported.assign((size_t)cfg->n_layers, false);
    m->nsplit = nsplit_for(cfg->max_ctx, cfg->attn_kv_heads, m->nsplit_w,
                           prop.multiProcessorCount < 256 ? prop.multiProcessorCount : 256);
    if (static_scratch_of(dev, &m->static_scratch) != hipSuccess) {
        delete m;
        return AW4_E_HIP;
    }
    m->static_need = static_step_bytes(m);
    // zero everything once (weights included) so unused tensors are defined
    if (launch_fill_zero(m->arena, need & ~uint64_t(3), m->stream) != hipSuccess) {
        delete m;
        return AW4_E_HIP;
    }
    *out = m;
    return AW4_OK;
}

void aw4_destroy(aw4_model* m) {
    if (!m) return;
    drop_graphs(m);
    delete m;
}

int aw4_tensor_shape(const aw4_model* mc, int32_t layer, int32_t kind, int64_t* rows, int64_t* cols) {
    aw4_model* m = const_cast<aw4_model*>(mc);
    if (check_model(m) || !rows || !cols) return AW4_E_INVAL;
    if (!cfg_tensor_shape(&m->cfg, layer, kind, rows, cols)) return fail(m, AW4_E_INVAL, "no such tensor");
    return AW4_OK;
}

int aw4_quantize_tensor(aw4_model* m, int32_t layer, int32_t kind, int64_t row0, int64_t nrows, const float* src) {
    if (check_model(m) || !src || nrows < 0) return AW4_E_INVAL;
    MatRef r;
    int rc = mat_ref(m, layer, kind, &r);
    if (rc) return rc;
    if (row0 < 0 || row0 + nrows > r.rows) return fail(m, AW4_E_INVAL, "row range outside the tensor");
    if (nrows == 0) return AW4_OK;
    if (r.i8) {
        HIPCHK(m, launch_quant_i8(src, nrows, r.cols, r.i8 + row0 * r.cols, r.scales + row0 * (r.cols / 32), m->stream));
    } else {
        HIPCHK(m, launch_quant_w4(src, nrows, r.cols, r.w4 + row0 * r.row_stride * (r.cols / 8),
                                  r.scales + row0 * r.row_stride * (r.cols / 32), r.row_stride, m->stream));
    }
    mark_rows(m, layer, kind, row0, nrows);
    drop_graphs(m);
    return AW4_OK;
}

int aw4_load_tensor(aw4_model* m, int32_t layer, int32_t kind, const void* host_codes, const uint16_t* host_scales) {
    if (check_model(m) || !host_codes || !host_scales) return AW4_E_INVAL;
    MatRef r;
    int rc = mat_ref(m, layer, kind, &r);
    if (rc) return rc;
    const int64_t G = r.cols / 32;
    HIPCHK(m, hipStreamSynchronize(m->stream));
    if (r.i8) {
        HIPCHK(m, hipMemcpy(r.i8, host_codes, (size_t)(r.rows * r.cols), hipMemcpyHostToDevice));
        HIPCHK(m, hipMemcpy(r.scales, host_scales, (size_t)(r.rows * G * 2), hipMemcpyHostToDevice));
        mark_rows(m, layer, kind, 0, r.rows);
        return AW4_OK;
    }
    const uint8_t* src = (const uint8_t*)host_codes;
    // pack on the host, copy row by row into the (possibly interleaved) GPU rows
    std::vector<uint32_t> buf((size_t)(r.rows * (r.cols / 8)));
    for (int64_t i = 0; i < r.rows; ++i) w4_logical_to_gpu(src + i * (r.cols / 2), r.cols, buf.data() + i * (r.cols / 8));
    HIPCHK(m, hipMemcpy2D(r.w4, (size_t)(r.row_stride * r.cols / 2), buf.data(), (size_t)(r.cols / 2),
                          (size_t)(r.cols / 2), (size_t)r.rows, hipMemcpyHostToDevice));
    HIPCHK(m, hipMemcpy2D(r.scales, (size_t)(r.row_stride * G * 2), host_scales, (size_t)(G * 2), (size_t)(G * 2),
                          (size_t)r.rows, hipMemcpyHostToDevice));
    mark_rows(m, layer, kind, 0, r.rows);
    drop_graphs(m);
    return AW4_OK;
}

int aw4_export_tensor(aw4_model* m, int32_t layer, int32_t kind, void* host_codes, uint16_t* host_scales) {
    if (check_model(m) || !host_codes || !host_scales) return AW4_E_INVAL;
    MatRef r;
    int rc = mat_ref(m, layer, kind, &r);
    if (rc) return rc;
    const int64_t G = r.cols / 32;
    HIPCHK(m, hipStreamSynchronize(m->stream));
    if (r.i8) {
        HIPCHK(m, hipMemcpy(host_codes, r.i8, (size_t)(r.rows * r.cols), hipMemcpyDeviceToHost));
        HIPCHK(m, hipMemcpy(host_scales, r.scales, (size_t)(r.rows * G * 2), hipMemcpyDeviceToHost));
        return AW4_OK;
    }
    std::vector<uint32_t> buf((size_t)(r.rows * (r.cols / 8)));
    HIPCHK(m, hipMemcpy2D(buf.data(), (size_t)(r.cols / 2), r.w4, (size_t)(r.row_stride * r.cols / 2),
                          (size_t)(r.cols / 2), (size_t)r.rows, hipMemcpyDeviceToHost));
    HIPCHK(m, hipMemcpy2D(host_scales, (size_t)(G * 2), r.scales, (size_t)(r.row_stride * G * 2), (size_t)(G * 2),
                          (size_t)r.rows, hipMemcpyDeviceToHost));
    uint8_t* dst = (uint8_t*)host_codes;
    for (int64_t i = 0; i < r.rows; ++i) w4_gpu_to_logical(buf.data() + i * (r.cols / 8), r.cols, dst + i * (r.cols / 2));
    return AW4_OK;
}

int aw4_set_vector(aw4_model* m, int32_t layer, int32_t kind, const float* vals, int32_t n) {
    if (check_model(m) || !vals) return AW4_E_INVAL;
    int64_t rows = 0, cols = 0;
    int rc = aw4_tensor_shape(m, layer, kind, &rows, &cols);
    if (rc) return rc;
    if (kind < 6 || kind == AW4_T_DRAFT_FUSE || kind == AW4_T_DRAFT_MAP || n != cols)
        return fail(m, AW4_E_INVAL, "vector length mismatch");
    float* dst = nullptr;
    if (kind == AW4_T_NORM_FINAL) dst = m->norm_final;
    else if (kind == AW4_T_DRAFT_NORM_EMB) dst = m->dn_emb;
    else if (kind == AW4_T_DRAFT_NORM_HID) dst = m->dn_hid;
    else if (kind == AW4_T_DRAFT_NORM_OUT) dst = m->dn_out;
    else if (kind == AW4_T_RHT_SIGNS) {
        for (int i = 0; i < n; ++i)
            if (vals[i] != 1.0f && vals[i] != -1.0f) return fail(m, AW4_E_INVAL, "rotation signs must be +-1");
        dst = m->signs;
    } else {
        LayerBufs& b = layer == m->cfg.n_layers ? m->D : m->L[layer];
        dst = kind == AW4_T_NORM_MIX ? b.norm_mix : kind == AW4_T_NORM_FFN ? b.norm_ffn
              : kind == AW4_T_NORM_GATED ? b.norm_gated : b.a_bias;
    }
    HIPCHK(m, hipStreamSynchronize(m->stream));
    HIPCHK(m, hipMemcpy(dst, vals, (size_t)n * 4, hipMemcpyHostToDevice));
    mark_rows(m, layer, kind, 0, 1);
    return AW4_OK;
}

int aw4_set_draft_map(aw4_model* m, const int32_t* ids, int32_t n) {
    if (check_model(m) || !ids) return AW4_E_INVAL;
    const aw4_config* c = &m->cfg;
    if (c->draft_vocab <= 0) return fail(m, AW4_E_STATE, "the model has no draft head");
    if (n != c->draft_vocab) return fail(m, AW4_E_INVAL, "the map must hold draft_vocab ids");
    std::vector<int32_t> sorted(ids, ids + n);
    std::sort(sorted.begin(), sorted.end());
    for (int i = 0; i < n; ++i)
        if (sorted[i] < 0 || sorted[i] >= c->vocab || (i > 0 && sorted[i] == sorted[i - 1]))
            return fail(m, AW4_E_INVAL, "map ids must be distinct and in [0, vocab)");
    std::vector<int32_t> rmap((size_t)c->vocab, -1);
    for (int i = 0; i < n; ++i) rmap[(size_t)sorted[i]] = i;
    HIPCHK(m, hipStreamSynchronize(m->stream));
    HIPCHK(m, hipMemcpy(m->dmap, sorted.data(), (size_t)n * 4, hipMemcpyHostToDevice));
    HIPCHK(m, hipMemcpy(m->drmap, rmap.data(), rmap.size() * 4, hipMemcpyHostToDevice));
    m->map_set = true;
    mark_rows(m, c->n_layers, AW4_T_DRAFT_MAP, 0, 1);
    return AW4_OK;
}

int aw4_test_fail_hip_call(int32_t n) {
    g_fail_countdown.store(n > 0 ? n : 0, std::memory_order_relaxed);
    return AW4_OK;
}

int aw4_check_blob(const aw4_config* cfg, const void* blob, uint64_t bytes) {
    if (check_config(cfg) || (!blob && bytes)) return AW4_E_INVAL;
    std::string why;
    return walk_blob(cfg, (const uint8_t*)blob, bytes, &why, nullptr);
}

int aw4_load_weights(aw4_model* m, const void* blob, uint64_t bytes) {
    if (check_model(m) || (!blob && bytes)) return AW4_E_INVAL;
    // the whole blob is checked first: a bad one changes nothing
    std::string why;
    if (walk_blob(&m->cfg, (const uint8_t*)blob, bytes, &why, nullptr)) return fail(m, AW4_E_FORMAT, why);
    int rc = walk_blob(&m->cfg, (const uint8_t*)blob, bytes, &why, [&](const BlobTensor& t) -> int {
        if (t.kind == AW4_T_DRAFT_MAP) {
            std::vector<int32_t> v((size_t)t.cols);
            memcpy(v.data(), t.payload, (size_t)t.cols * 4);
            return aw4_set_draft_map(m, v.data(), (int32_t)t.cols);
        }
        if (is_matrix_kind(t.kind)) {
            const uint64_t cb = t.kind == AW4_T_LM_HEAD ? (uint64_t)(t.rows * t.cols) : (uint64_t)(t.rows * t.cols / 2);
            std::vector<uint16_t> sc((size_t)(t.rows * (t.cols / 32)));
            memcpy(sc.data(), t.payload + cb, sc.size() * 2);
            return aw4_load_tensor(m, t.layer, t.kind, t.payload, sc.data());
        }
        std::vector<float> v((size_t)t.cols);
        memcpy(v.data(), t.payload, (size_t)t.cols * 4);
        return aw4_set_vector(m, t.layer, t.kind, v.data(), (int32_t)t.cols);
    });
    return rc;
}

int aw4_reset(aw4_model* m) {
    if (check_model(m)) return AW4_E_INVAL;
    HIPCHK(m, launch_fill_zero(m->arena + m->state_off, m->state_bytes * (uint64_t)m->max_batch, m->stream));
    HIPCHK(m, launch_set_ctl(m->ctl, 0, 0, 0, m->stream));
    HIPCHK(m, launch_set_dpos(m->ctl, 0, m->stream));
    m->host_pos = 0;
    m->host_dpos = 0;
    m->pend_src = 0;
    for (int b = 0; b < 4; ++b) m->seq_pos[b] = m->seq_dpos[b] = 0;
    m->win_fresh.assign(m->win_fresh.size(), true);
    return AW4_OK;
}

int aw4_set_graph(aw4_model* m, int32_t enable) {
    if (check_model(m)) return AW4_E_INVAL;
    m->use_graph = enable != 0;
    if (!m->use_graph) drop_graphs(m);
    return AW4_OK;
}

int aw4_get_pos(aw4_model* m, int32_t* pos) {
    if (check_model(m) || !pos) return AW4_E_INVAL;
    *pos = m->host_pos;
    return AW4_OK;
}

int aw4_set_pos(aw4_model* m, int32_t pos) {
    if (check_model(m)) return AW4_E_INVAL;
    if (pos < 0 || pos > m->cfg.max_ctx) return fail(m, AW4_E_CTX_FULL, "position outside [0, max_ctx]");
    HIPCHK(m, launch_set_ctl(m->ctl, pos, -1, -1, m->stream));
    // moving back leaves ring slots holding positions after the new one
    if (m->cfg.kv_window > 0 && pos < m->host_pos)
        for (int l = 0; l < m->cfg.n_layers; ++l)
            if (m->L[l].type == 'A' && !m->win_imported[(size_t)l]) m->win_fresh[(size_t)l] = false;
    m->host_pos = pos;
    m->pend_src = 0;
    return AW4_OK;
}

int aw4_select_sequence(aw4_model* m, int32_t s) {
    if (check_model(m)) return AW4_E_INVAL;
    if (s < 0 || s >= m->max_batch) return fail(m, AW4_E_INVAL, "sequence outside [0, max_batch)");
    if (s == m->seq) return AW4_OK;
    m->seq_pos[m->seq] = m->host_pos;
    m->seq_dpos[m->seq] = m->host_dpos;
    shift_state(m, s - m->seq);
    m->seq = s;
    m->host_pos = m->seq_pos[s];
    m->host_dpos = m->seq_dpos[s];
    HIPCHK(m, launch_set_ctl(m->ctl, m->host_pos, -1, -1, m->stream));
    HIPCHK(m, launch_set_dpos(m->ctl, m->host_dpos, m->stream));
    m->pend_src = 0;
    drop_graphs(m);   // the captured step holds the previous sequence's state pointers
    return AW4_OK;
}

int aw4_decode_batch(aw4_model* m, const int32_t* host_tokens, int32_t B, int32_t* host_argmax) {
    if (check_model(m) || !host_tokens || !host_argmax) return AW4_E_INVAL;
    const aw4_config* c = &m->cfg;
    if (c->vocab <= 0) return fail(m, AW4_E_STATE, "decode_batch needs a vocabulary");
    if (need_weights(m)) return AW4_E_STATE;
    if (B < 1 || B > m->max_batch) return fail(m, AW4_E_INVAL, "batch must be in [1, max_batch]");
    if (c->kv_window > 0) return fail(m, AW4_E_INVAL, "batch decode does not read a recent window");
    if (B == 1 && m->seq == 0) {
        // one sequence, the selected one: the single-token step computes the
        // same thing with the kernels built for one input vector
        int rc = aw4_decode_step(m, host_tokens[0], nullptr, host_argmax);
        if (rc) return rc;
        m->seq_pos[0] = m->host_pos;
        m->pend_src = 0;
        return AW4_OK;
    }
    m->seq_pos[m->seq] = m->host_pos;
    int32_t tok[4] = {0, 0, 0, 0}, pos[4] = {0, 0, 0, 0};
    for (int b = 0; b < B; ++b) {
        if (host_tokens[b] < 0 || host_tokens[b] >= c->vocab) return fail(m, AW4_E_TOKEN, "token out of range");
        if (m->seq_pos[b] + 1 > c->max_ctx) return fail(m, AW4_E_CTX_FULL, "context full");
        tok[b] = host_tokens[b];
        pos[b] = m->seq_pos[b];
    }
    hipStream_t s = m->stream;
    // tokens and positions go to the control block; the step itself reads
    // them there, so one captured graph per batch size serves every call
    HIPCHK(m, launch_set_batch(m->ctl, tok, pos, s));
    if (m->use_graph) {
        hipGraphExec_t* ge = &m->g_batch[B];
        if (!*ge) {
            hipGraph_t g = nullptr;
            HIPCHK_RAW(m, hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
            int rc = enqueue_batch_step(m, B);
            hipError_t e = hipStreamEndCapture(s, &g);
            if (rc) {
                if (g) (void)hipGraphDestroy(g);
                return rc;
            }
            if (e != hipSuccess) return fail(m, AW4_E_HIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(e));
            e = hipGraphInstantiate(ge, g, nullptr, nullptr, 0);
            (void)hipGraphDestroy(g);
            if (e != hipSuccess) {
                *ge = nullptr;
                return fail(m, AW4_E_HIP, std::string("hipGraphInstantiate: ") + hipGetErrorString(e));
            }
        }
        HIPCHK(m, hipGraphLaunch(*ge, s));
    } else {
        int rc = enqueue_batch_step(m, B);
        if (rc) return rc;
    }
    int32_t am[4];
    HIPCHK(m, hipMemcpyAsync(am, &m->ctl->vargmax[0], 4 * sizeof(int32_t), hipMemcpyDeviceToHost, s));
    HIPCHK(m, hipStreamSynchronize(s));
    for (int b = 0; b < B; ++b) {
        host_argmax[b] = am[b];
        m->seq_pos[b] += 1;
    }
    m->host_pos = m->seq_pos[m->seq];
    HIPCHK(m, launch_set_ctl(m->ctl, m->host_pos, -1, -1, s));
    m->pend_src = 0;
    return AW4_OK;
}

int aw4_get_draft_pos(aw4_model* m, int32_t* dpos) {
    if (check_model(m) || !dpos) return AW4_E_INVAL;
    if (m->cfg.draft_vocab <= 0) return fail(m, AW4_E_STATE, "the model has no draft head");
    *dpos = m->host_dpos;
    return AW4_OK;
}

int aw4_set_draft_pos(aw4_model* m, int32_t dpos) {
    if (check_model(m)) return AW4_E_INVAL;
    if (m->cfg.draft_vocab <= 0) return fail(m, AW4_E_STATE, "the model has no draft head");
    if (dpos < 0 || dpos > m->cfg.max_ctx) return fail(m, AW4_E_CTX_FULL, "draft length outside [0, max_ctx]");
    HIPCHK(m, launch_set_dpos(m->ctl, dpos, m->stream));
    m->host_dpos = dpos;
    return AW4_OK;
}

int aw4_draft(aw4_model* m, int32_t t0, int32_t k, float temperature, const float* host_u, float* dev_q,
              float* dev_scores, int32_t* host_drafts) {
    if (check_model(m) || !host_drafts) return AW4_E_INVAL;
    const aw4_config* c = &m->cfg;
    if (c->draft_vocab <= 0) return fail(m, AW4_E_STATE, "the model has no draft head");
    if (!m->map_set) return fail(m, AW4_E_STATE, "no vocabulary map has been set");
    if (need_weights(m)) return AW4_E_STATE;
    if (k < 1 || k > 3 || k + 1 > c->max_verify) return fail(m, AW4_E_INVAL, "k must be in [1, min(3, max_verify - 1)]");
    if (t0 < 0 || t0 >= c->vocab) return fail(m, AW4_E_TOKEN, "token out of range");
    if (!(temperature >= 0.f) || !std::isfinite(temperature)) return fail(m, AW4_E_INVAL, "temperature must be >= 0");
    if (temperature > 0.f) {
        if (!host_u) return fail(m, AW4_E_INVAL, "sampling needs one uniform per draft");
        for (int i = 0; i < k; ++i)
            if (!(host_u[i] >= 0.f && host_u[i] < 1.f)) return fail(m, AW4_E_INVAL, "uniforms must lie in [0, 1)");
    }
    if (m->pend_src == 0)
        return fail(m, AW4_E_STATE, "no committed hidden state to draft from (decode, prefill or verify first)");
    const int M = m->pend_n + 1;
    if ((int64_t)m->host_dpos + M + (k - 1) > c->max_ctx) return fail(m, AW4_E_CTX_FULL, "draft cache full");
    int32_t tok[4] = {0, 0, 0, 0};
    float u[4] = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < m->pend_n; ++i) tok[i] = m->pend_tok[i];
    tok[M - 1] = t0;
    for (int i = 0; i < k && temperature > 0.f; ++i) u[i] = host_u[i];
    const int H = c->hidden;
    const bool q_out = temperature > 0.f && dev_q;
    HIPCHK(m, launch_set_draft(m->ctl, tok, u, m->stream));
    // the pending entries and t0's entry, committed; draft 1 from the last row
    int rc = enqueue_draft_block(m, M, &m->ctl->dtok[0], m->pend_src == 1 ? m->x : m->vx, H, 0);
    if (rc) return rc;
    rc = enqueue_draft_select(m, M - 1, 0, M, temperature, q_out ? dev_q : nullptr, dev_scores);
    if (rc) return rc;
    // drafts 2..k from the block's own output and the previous draft, in entries
    // past the committed length
    for (int j = 1; j < k; ++j) {
        rc = enqueue_draft_block(m, 1, &m->ctl->dout[j - 1], m->xd + (j == 1 ? (int64_t)(M - 1) * H : 0), H, j - 1);
        if (rc) return rc;
        rc = enqueue_draft_select(m, 0, j, 0, temperature, q_out ? dev_q + (int64_t)j * c->vocab : nullptr,
                                  dev_scores ? dev_scores + (int64_t)j * c->draft_vocab : nullptr);
        if (rc) return rc;
    }
    int32_t out[4];
    HIPCHK(m, hipMemcpyAsync(out, &m->ctl->dout[0], 4 * sizeof(int32_t), hipMemcpyDeviceToHost, m->stream));
    HIPCHK(m, hipStreamSynchronize(m->stream));
    for (int i = 0; i < k; ++i) host_drafts[i] = out[i];
    m->host_dpos += M;
    m->pend_src = 0;
    m->pend_n = 0;
    return AW4_OK;
}

int aw4_prefill(aw4_model* m, const int32_t* tokens, int32_t n, float* dev_logits) {
    if (check_model(m) || (!tokens && n > 0) || n < 0) return AW4_E_INVAL;
    if (m->cfg.vocab <= 0) return fail(m, AW4_E_STATE, "prefill needs a vocabulary");
    if (need_weights(m) || need_fresh_window(m)) return AW4_E_STATE;
    if ((int64_t)m->host_pos + n > m->cfg.max_ctx) return fail(m, AW4_E_CTX_FULL, "prompt exceeds max_ctx");
    for (int i = 0; i < n; ++i)
        if (tokens[i] < 0 || tokens[i] >= m->cfg.vocab) return fail(m, AW4_E_TOKEN, "prompt token out of range");
    const bool feed = m->cfg.draft_vocab > 0;
    if (feed && n > 0 && (int64_t)m->host_dpos + n - 1 > m->cfg.max_ctx)
        return fail(m, AW4_E_CTX_FULL, "prompt exceeds the draft head's cache");
    if (n == 0) return AW4_OK;
    if (m->pchunk > 0) {
        int rc = enqueue_prefill_chunked(m, tokens, n, dev_logits != nullptr);
        if (rc) return rc;
    } else {
        // token by token through the decode step
        for (int i = 0; i < n; ++i) {
            HIPCHK(m, launch_set_token(m->ctl, tokens[i], m->stream));
            const bool last = i == n - 1;
            int rc = run_step(m, last && dev_logits != nullptr);
            if (rc) return rc;
            m->host_pos += 1;
            if (feed && !last) {
                // the draft head's entry of this position: (its hidden state, the next prompt token)
                const int32_t tok[4] = {tokens[i + 1], 0, 0, 0};
                const float u[4] = {0.f, 0.f, 0.f, 0.f};
                HIPCHK(m, launch_set_draft(m->ctl, tok, u, m->stream));
                rc = enqueue_draft_block(m, 1, &m->ctl->dtok[0], m->x, m->cfg.hidden, 0);
                if (rc) return rc;
                m->host_dpos += 1;
                HIPCHK(m, launch_set_dpos(m->ctl, m->host_dpos, m->stream));
            }
        }
    }
    m->pend_src = 1;
    m->pend_n = 0;
    if (dev_logits)
        HIPCHK(m, hipMemcpyAsync(dev_logits, m->logits, (size_t)m->cfg.vocab * 4, hipMemcpyDeviceToDevice, m->stream));
    return AW4_OK;
}

int aw4_set_prefill_chunk(aw4_model* m, int32_t n) {
    if (check_model(m)) return AW4_E_INVAL;
    if (n < 0 || n > m->pchunk_max)
        return fail(m, AW4_E_INVAL, "chunk must be in [0, " + std::to_string(m->pchunk_max) + "]");
    m->pchunk = n;
    return AW4_OK;
}

int aw4_decode_step(aw4_model* m, int32_t token, float* dev_logits, int32_t* host_argmax) {
    if (check_model(m)) return AW4_E_INVAL;
    if (m->cfg.vocab <= 0) return fail(m, AW4_E_STATE, "decode_step needs a vocabulary");
    if (need_weights(m) || need_fresh_window(m)) return AW4_E_STATE;
    if (token < 0 || token >= m->cfg.vocab) return fail(m, AW4_E_TOKEN, "token out of range");
    if (m->host_pos + 1 > m->cfg.max_ctx) return fail(m, AW4_E_CTX_FULL, "context full");
    HIPCHK(m, launch_set_token(m->ctl, token, m->stream));
    int rc = run_step(m, true);
    if (rc) return rc;
    m->host_pos += 1;
    m->pend_src = 1;
    m->pend_n = 0;
    if (dev_logits)
        HIPCHK(m, hipMemcpyAsync(dev_logits, m->logits, (size_t)m->cfg.vocab * 4, hipMemcpyDeviceToDevice, m->stream));
    if (host_argmax) {
        HIPCHK(m, hipMemcpyAsync(host_argmax, &m->ctl->argmax, 4, hipMemcpyDeviceToHost, m->stream));
        HIPCHK(m, hipStreamSynchronize(m->stream));
    }
    return AW4_OK;
}

int aw4_decode_step_static(aw4_model* m, int32_t token, float* dev_logits, int32_t* host_argmax) {
    if (check_model(m)) return AW4_E_INVAL;
    if (m->cfg.vocab <= 0) return fail(m, AW4_E_STATE, "decode_step needs a vocabulary");
    if (m->static_need > kStaticScratchBytes)
        return fail(m, AW4_E_INVAL, "the step needs " + std::to_string(m->static_need) +
                                        " bytes of static scratch; the library holds " +
                                        std::to_string(kStaticScratchBytes));
    if (need_weights(m) || need_fresh_window(m)) return AW4_E_STATE;
    if (token < 0 || token >= m->cfg.vocab) return fail(m, AW4_E_TOKEN, "token out of range");
    if (m->host_pos + 1 > m->cfg.max_ctx) return fail(m, AW4_E_CTX_FULL, "context full");
    HIPCHK(m, launch_set_token(m->ctl, token, m->stream));
    // the same step with its partials in the static scratch (one token's
    // rows), launched kernel by kernel: no graph of its own, so a caller may
    // capture these launches into its own graph
    const uint64_t part_bytes = m->static_need - 2 * (((uint64_t)m->nhead_blocks * 4 + 255) & ~uint64_t(255));
    m->step_part = (float*)m->static_scratch;
    m->step_prow = m->cfg.attn_q_heads;
    m->step_pv = (float*)(m->static_scratch + part_bytes);
    m->step_pi = (int32_t*)(m->static_scratch + part_bytes + (((uint64_t)m->nhead_blocks * 4 + 255) & ~uint64_t(255)));
    const int rc = enqueue_step(m, true);
    m->step_part = m->part;
    m->step_prow = kSweepRows * m->cfg.attn_q_heads;
    m->step_pv = m->pv;
    m->step_pi = m->pi;
    if (rc) return rc;
    m->host_pos += 1;
    m->pend_src = 1;
    m->pend_n = 0;
    if (dev_logits)
        HIPCHK(m, hipMemcpyAsync(dev_logits, m->logits, (size_t)m->cfg.vocab * 4, hipMemcpyDeviceToDevice, m->stream));
    if (host_argmax) {
        HIPCHK(m, hipMemcpyAsync(host_argmax, &m->ctl->argmax, 4, hipMemcpyDeviceToHost, m->stream));
        HIPCHK(m, hipStreamSynchronize(m->stream));
    }
    return AW4_OK;
}

int aw4_decode_greedy(aw4_model* m, int32_t first_token, int32_t n_steps, int32_t* host_out) {
    if (check_model(m) || n_steps < 0 || (!host_out && n_steps > 0)) return AW4_E_INVAL;
    if (m->cfg.vocab <= 0) return fail(m, AW4_E_STATE, "decode_greedy needs a vocabulary");
    if (need_weights(m) || need_fresh_window(m)) return AW4_E_STATE;
    if (first_token < 0 || first_token >= m->cfg.vocab) return fail(m, AW4_E_TOKEN, "token out of range");
    if ((int64_t)m->host_pos + n_steps > m->cfg.max_ctx) return fail(m, AW4_E_CTX_FULL, "context full");
    int done = 0;
    int32_t tok = first_token;
    while (done < n_steps) {
        const int chunk = n_steps - done < m->ring_cap ? n_steps - done : m->ring_cap;
        HIPCHK(m, launch_set_ctl(m->ctl, -1, tok, 0, m->stream));
        for (int i = 0; i < chunk; ++i) {
            int rc = run_step(m, true);
            if (rc) return rc;
            m->host_pos += 1;
        }
        HIPCHK(m, hipMemcpyAsync(host_out + done, m->ring, (size_t)chunk * 4, hipMemcpyDeviceToHost, m->stream));
        HIPCHK(m, hipStreamSynchronize(m->stream));
        done += chunk;
        tok = host_out[done - 1];
        m->pend_src = 1;
        m->pend_n = 0;
    }
    return AW4_OK;
}

int aw4_verify_k(aw4_model* m, const int32_t* host_tokens, int32_t k, const float* dev_q, const float* host_u,
                 float temperature, int32_t* host_out, int32_t* host_n_out) {
    if (check_model(m) || !host_tokens || !host_out || !host_n_out) return AW4_E_INVAL;
    const aw4_config* c = &m->cfg;
    if (c->vocab <= 0) return fail(m, AW4_E_STATE, "verify_k needs a vocabulary");
    if (need_weights(m)) return AW4_E_STATE;
    if (c->kv_window > 0) return fail(m, AW4_E_INVAL, "verify_k does not read a recent window");
    if (c->kv_format != 0) return fail(m, AW4_E_INVAL, "verify_k reads the int8 / 3-bit cache only (kv_format 0)");
    if (k < 0 || k + 1 > c->max_verify) return fail(m, AW4_E_INVAL, "k must be in [0, max_verify - 1]");
    if (!(temperature >= 0.f) || !std::isfinite(temperature)) return fail(m, AW4_E_INVAL, "temperature must be >= 0");
    if (temperature > 0.f && (!host_u || (k > 0 && !dev_q)))
        return fail(m, AW4_E_INVAL, "sampling needs uniforms and draft probabilities");
    for (int i = 0; i <= k; ++i)
        if (host_tokens[i] < 0 || host_tokens[i] >= c->vocab) return fail(m, AW4_E_TOKEN, "token out of range");
    if (host_u)
        for (int i = 0; i <= k; ++i)
            if (!(host_u[i] >= 0.f && host_u[i] < 1.f)) return fail(m, AW4_E_INVAL, "uniforms must lie in [0, 1)");
    if ((int64_t)m->host_pos + k + 1 > c->max_ctx) return fail(m, AW4_E_CTX_FULL, "context full");
    int32_t tok[4] = {0, 0, 0, 0};
    float u[4] = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i <= k; ++i) {
        tok[i] = host_tokens[i];
        if (host_u) u[i] = host_u[i];
    }
    // the uniform of the final draw is u[k]
    HIPCHK(m, launch_set_verify(m->ctl, tok, u, m->stream));
    int rc = enqueue_verify(m, k + 1, k, dev_q, temperature);
    if (rc) return rc;
    int32_t res[8];
    HIPCHK(m, hipMemcpyAsync(res, &m->ctl->vout[0], 4 * sizeof(int32_t), hipMemcpyDeviceToHost, m->stream));
    HIPCHK(m, hipMemcpyAsync(res + 4, &m->ctl->vn_acc, 4 * sizeof(int32_t), hipMemcpyDeviceToHost, m->stream));
    HIPCHK(m, hipStreamSynchronize(m->stream));
    const int n_out = res[5];
    if (n_out < 1 || n_out > k + 1) return fail(m, AW4_E_HIP, "verify produced an invalid token count");
    for (int i = 0; i < n_out; ++i) host_out[i] = res[i];
    *host_n_out = n_out;
    m->host_pos += res[6];
    // the accepted positions' hidden states (verify rows 0 .. n_out - 1) wait for
    // the next draft call, with the drafts that followed them
    m->pend_src = 2;
    m->pend_n = n_out - 1;
    for (int i = 0; i + 1 < n_out; ++i) m->pend_tok[i] = host_tokens[i + 1];
    return AW4_OK;
}

int aw4_decode_hidden(aw4_model* m, const float* dev_in, float* dev_out) {
    if (check_model(m) || !dev_in || !dev_out) return AW4_E_INVAL;
    if (need_weights(m) || need_fresh_window(m)) return AW4_E_STATE;
    if (m->host_pos + 1 > m->cfg.max_ctx) return fail(m, AW4_E_CTX_FULL, "context full");
    if (dev_in != m->x) HIPCHK(m, launch_copy_f32(m->x, dev_in, m->cfg.hidden, m->stream));
    int rc = enqueue_layers(m);
    if (rc) return rc;
    HIPCHK(m, launch_advance(m->ctl, m->stream));
    if (dev_out != m->x) HIPCHK(m, launch_copy_f32(dev_out, m->x, m->cfg.hidden, m->stream));
    m->host_pos += 1;
    m->pend_src = 0;
    return AW4_OK;
}

int aw4_read_hidden(aw4_model* m, float* host_x) {
    if (check_model(m) || !host_x) return AW4_E_INVAL;
    HIPCHK(m, hipMemcpyAsync(host_x, m->x, (size_t)m->cfg.hidden * 4, hipMemcpyDeviceToHost, m->stream));
    HIPCHK(m, hipStreamSynchronize(m->stream));
    return AW4_OK;
}

int aw4_time_phase(aw4_model* m, int32_t phase, int32_t reps, float* avg_us, uint64_t* bytes_per_launch) {
    if (check_model(m) || reps < 1 || !avg_us || !bytes_per_launch) return AW4_E_INVAL;
    if (phase < 0 || phase > AW4_PHASE_PREFILL_GATE_UP) return fail(m, AW4_E_INVAL, "unknown phase");
    if (need_weights(m)) return AW4_E_STATE;
    hipEvent_t e0, e1;
    HIPCHK(m, hipEventCreate(&e0));
    HIPCHK(m, hipEventCreate(&e1));
    uint64_t bytes = 0;
    const int L = m->cfg.n_layers;
    // round robin over the layers so that consecutive launches stream different
    // weights (a single layer's matrices would stay in the 256 MB last-level cache)
    for (int i = 0; i < L && i < reps; ++i) {
        int rc = enqueue_phase(m, phase, i % L, &bytes);
        if (rc) return rc;
    }
    // the timed launches run as one captured graph, the way the decode step
    // runs them (eager launches of the large grids spent several microseconds
    // each on launch overhead); without graphs, and for the prefill GEMM (1.4 ms
    // a launch), they are launched one by one
    // The decode GEMV phases are timed in context: each timed launch follows a
    // launch of the GEMV that precedes it in the decode step (down before
    // gate/up and before the in-projection, gate/up before down), and a pair
    // of events inside the graph brackets the timed launch alone.  Back to
    // back, launches of one kernel ran 10-15% slower than the same kernel
    // inside the decode step.
    if (m->use_graph && phase <= AW4_PHASE_MIX_IN) {
        const int cphase = phase == AW4_PHASE_FFN_DOWN ? AW4_PHASE_FFN_GATE_UP : AW4_PHASE_FFN_DOWN;
        std::vector<hipEvent_t> ev(2 * (size_t)reps, nullptr);
        bool ok = true;
        for (auto& e : ev) ok = ok && hipEventCreate(&e) == hipSuccess;
        hipGraph_t g = nullptr;
        hipGraphExec_t gx = nullptr;
        if (ok) ok = hipStreamBeginCapture(m->stream, hipStreamCaptureModeThreadLocal) == hipSuccess;
        if (ok) {
            uint64_t cb = 0;
            for (int i = 0; i < reps && ok; ++i) {
                ok = enqueue_phase(m, cphase, (i + L - 1) % L, &cb) == AW4_OK &&
                     hipEventRecord(ev[2 * i], m->stream) == hipSuccess &&
                     enqueue_phase(m, phase, i % L, &bytes) == AW4_OK &&
                     hipEventRecord(ev[2 * i + 1], m->stream) == hipSuccess;
            }
            const bool ended = hipStreamEndCapture(m->stream, &g) == hipSuccess;
            ok = ok && ended && g && hipGraphInstantiate(&gx, g, nullptr, nullptr, 0) == hipSuccess;
            if (g) (void)hipGraphDestroy(g);
        }
        float tot = 0.f;
        if (ok) ok = hipGraphLaunch(gx, m->stream) == hipSuccess &&   // untimed pass
                     hipGraphLaunch(gx, m->stream) == hipSuccess && hipStreamSynchronize(m->stream) == hipSuccess;
        for (int i = 0; i < reps && ok; ++i) {
            float ms = 0.f;
            ok = hipEventElapsedTime(&ms, ev[2 * i], ev[2 * i + 1]) == hipSuccess;
            tot += ms;
        }
        if (gx) (void)hipGraphExecDestroy(gx);
        for (auto& e : ev)
            if (e) (void)hipEventDestroy(e);
        (void)hipGetLastError();   // a failed attempt falls back to the timing below
        if (ok) {
            (void)hipEventDestroy(e0);
            (void)hipEventDestroy(e1);
            *avg_us = tot * 1000.f / (float)reps;
            *bytes_per_launch = bytes;
            return AW4_OK;
        }
    }
    hipGraphExec_t ge = nullptr;
    if (m->use_graph && phase != AW4_PHASE_PREFILL_GATE_UP) {
        hipGraph_t g = nullptr;
        HIPCHK_RAW(m, hipStreamBeginCapture(m->stream, hipStreamCaptureModeThreadLocal));
        for (int i = 0; i < reps; ++i) {
            int rc = enqueue_phase(m, phase, i % L, &bytes);
            if (rc) {
                (void)hipStreamEndCapture(m->stream, &g);
                if (g) (void)hipGraphDestroy(g);
                return rc;
            }
        }
        HIPCHK(m, hipStreamEndCapture(m->stream, &g));
        hipError_t e = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
        (void)hipGraphDestroy(g);
        if (e != hipSuccess) return fail(m, AW4_E_HIP, std::string("phase graph: ") + hipGetErrorString(e));
        HIPCHK(m, hipGraphLaunch(ge, m->stream));   // untimed pass
    }
    HIPCHK(m, hipEventRecord(e0, m->stream));
    if (ge) {
        HIPCHK(m, hipGraphLaunch(ge, m->stream));
    } else {
        for (int i = 0; i < reps; ++i) {
            int rc = enqueue_phase(m, phase, i % L, &bytes);
            if (rc) return rc;
        }
    }
    HIPCHK(m, hipEventRecord(e1, m->stream));
    HIPCHK(m, hipEventSynchronize(e1));
    if (ge) (void)hipGraphExecDestroy(ge);
    float ms = 0.f;
    HIPCHK(m, hipEventElapsedTime(&ms, e0, e1));
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    *avg_us = ms * 1000.f / (float)reps;
    *bytes_per_launch = bytes;
    return AW4_OK;
}

int aw4_export_state_gdn(aw4_model* m, int32_t layer, float* host_S) {
    if (check_model(m) || !host_S || layer < 0 || layer >= m->cfg.n_layers || m->L[layer].type != 'G')
        return fail(m, AW4_E_INVAL, "not a GDN layer");
    const aw4_config* c = &m->cfg;
    const size_t n = (size_t)c->gdn_v_heads * c->gdn_head_dim * c->gdn_head_dim;
    HIPCHK(m, hipStreamSynchronize(m->stream));
    HIPCHK(m, hipMemcpy(host_S, m->L[layer].S, n * 4, hipMemcpyDeviceToHost));
    return AW4_OK;
}

int aw4_import_state_gdn(aw4_model* m, int32_t layer, const float* host_S) {
    if (check_model(m) || !host_S || layer < 0 || layer >= m->cfg.n_layers || m->L[layer].type != 'G')
        return fail(m, AW4_E_INVAL, "not a GDN layer");
    const aw4_config* c = &m->cfg;
    const size_t n = (size_t)c->gdn_v_heads * c->gdn_head_dim * c->gdn_head_dim;
    HIPCHK(m, hipStreamSynchronize(m->stream));
    HIPCHK(m, hipMemcpy(m->L[layer].S, host_S, n * 4, hipMemcpyHostToDevice));
    return AW4_OK;
}

int aw4_export_state_kv(aw4_model* m, int32_t layer, int32_t npos, int8_t* kc, uint16_t* ks, int8_t* vc,
                        uint16_t* vs) {
    LayerBufs* lb = kv_layer(m, layer);
    if (check_model(m) || !kc || !ks || !vc || !vs || !lb) return fail(m, AW4_E_INVAL, "not an attention layer");
    const aw4_config* c = &m->cfg;
    if (npos < 0 || npos > c->max_ctx) return fail(m, AW4_E_INVAL, "npos outside [0, max_ctx]");
    const int nkv = c->attn_kv_heads, d = c->attn_head_dim, NG = d / 32;
    const int fmt = layer == c->n_layers ? 0 : c->kv_format;   // the draft head's cache is format 0
    const int FB = fmt == 1 ? 4 : 3, VW = FB * NG, KR = fmt == 1 ? d / 2 : d;
    LayerBufs& b = *lb;
    HIPCHK(m, hipStreamSynchronize(m->stream));
    std::vector<int8_t> k((size_t)npos * KR);
    std::vector<uint16_t> s1((size_t)npos * NG), s2((size_t)npos * NG);
    std::vector<uint32_t> v((size_t)npos * VW + 1);
    for (int j = 0; j < nkv && npos > 0; ++j) {
        const int64_t hb = (int64_t)j * c->max_ctx;
        HIPCHK(m, hipMemcpy(k.data(), b.kc + hb * KR, (size_t)npos * KR, hipMemcpyDeviceToHost));
        HIPCHK(m, hipMemcpy(s1.data(), b.ks + hb * NG, s1.size() * 2, hipMemcpyDeviceToHost));
        HIPCHK(m, hipMemcpy(s2.data(), b.vs + hb * NG, s2.size() * 2, hipMemcpyDeviceToHost));
        HIPCHK(m, hipMemcpy(v.data(), b.vc + hb * VW, (size_t)npos * VW * 4, hipMemcpyDeviceToHost));
        for (int t = 0; t < npos; ++t) {
            const int64_t lo = ((int64_t)t * nkv + j);
            const int8_t* kr = k.data() + (size_t)t * KR;
            const uint32_t* rec = v.data() + (size_t)t * VW;
            for (int e = 0; e < d; ++e) {
                if (fmt == 1) {
                    const int kb = kv_key_nib_bit(e, d);
                    kc[lo * d + e] = (int8_t)((int)((((const uint32_t*)kr)[kb >> 5] >> (kb & 31)) & 15u) - 8);
                    const uint32_t f = kv_value_field(rec, VW, kv_value_bit_fb(e, d, 4), 4);
                    vc[lo * d + e] = (int8_t)((int)f - 8);
                } else {
                    kc[lo * d + e] = (int8_t)((int)(uint8_t)kr[kv_key_byte(e, d)] - 128);
                    const uint32_t f = kv_value_field(rec, VW, kv_value_bit(e, d));
                    vc[lo * d + e] = (int8_t)(fmt == 2 ? lm_code(f) : (int)f - 4);
                }
            }
            memcpy(ks + lo * NG, s1.data() + (size_t)t * NG, (size_t)NG * 2);
            memcpy(vs + lo * NG, s2.data() + (size_t)t * NG, (size_t)NG * 2);
        }
    }
    return AW4_OK;
}

int aw4_import_state_kv(aw4_model* m, int32_t layer, int32_t npos, const int8_t* kc, const uint16_t* ks,
                        const int8_t* vc, const uint16_t* vs) {
    LayerBufs* lb = kv_layer(m, layer);
    if (check_model(m) || !kc || !ks || !vc || !vs || !lb) return fail(m, AW4_E_INVAL, "not an attention layer");
    const aw4_config* c = &m->cfg;
    if (npos < 0 || npos > c->max_ctx) return fail(m, AW4_E_INVAL, "npos outside [0, max_ctx]");
    const int nkv = c->attn_kv_heads, d = c->attn_head_dim, NG = d / 32;
    const int fmt = layer == c->n_layers ? 0 : c->kv_format;   // the draft head's cache is format 0
    const int FB = fmt == 1 ? 4 : 3, VW = FB * NG, KR = fmt == 1 ? d / 2 : d;
    const int vlo = fmt == 1 ? -7 : fmt == 2 ? 0 : -3, vhi = fmt == 1 ? 7 : fmt == 2 ? 7 : 3;
    for (int64_t i = 0; i < (int64_t)npos * nkv * d; ++i) {
        if (vc[i] < vlo || vc[i] > vhi)
            return fail(m, AW4_E_INVAL, "V codes must be in " + std::to_string(vlo) + ".." + std::to_string(vhi));
        if (fmt == 1 && (kc[i] < -7 || kc[i] > 7)) return fail(m, AW4_E_INVAL, "K codes must be in -7..7");
    }
    LayerBufs& b = *lb;
    HIPCHK(m, hipStreamSynchronize(m->stream));
    std::vector<int8_t> k((size_t)npos * KR);
    std::vector<uint16_t> s1((size_t)npos * NG), s2((size_t)npos * NG);
    std::vector<uint32_t> v((size_t)npos * VW);
    for (int j = 0; j < nkv && npos > 0; ++j) {
        std::fill(v.begin(), v.end(), 0u);
        std::fill(k.begin(), k.end(), (int8_t)0);
        for (int t = 0; t < npos; ++t) {
            const int64_t lo = ((int64_t)t * nkv + j);
            int8_t* kr = k.data() + (size_t)t * KR;
            uint32_t* rec = v.data() + (size_t)t * VW;
            for (int e = 0; e < d; ++e) {
                uint32_t n;
                int bit;
                if (fmt == 1) {
                    const int kb = kv_key_nib_bit(e, d);
                    ((uint32_t*)kr)[kb >> 5] |= ((uint32_t)(kc[lo * d + e] + 8) & 15u) << (kb & 31);
                    n = (uint32_t)(vc[lo * d + e] + 8) & 15u;
                    bit = kv_value_bit_fb(e, d, 4);
                } else {
                    kr[kv_key_byte(e, d)] = (int8_t)(uint8_t)((int)kc[lo * d + e] + 128);
                    n = fmt == 2 ? lm_field(vc[lo * d + e]) : (uint32_t)(vc[lo * d + e] + 4) & 7u;
                    bit = kv_value_bit(e, d);
                }
                const int wi = bit >> 5, off = bit & 31;
                rec[wi] |= n << off;
                if (off > 32 - FB) rec[wi + 1] |= n >> (32 - off);
            }
            memcpy(s1.data() + (size_t)t * NG, ks + lo * NG, (size_t)NG * 2);
            memcpy(s2.data() + (size_t)t * NG, vs + lo * NG, (size_t)NG * 2);
        }
        const int64_t hb = (int64_t)j * c->max_ctx;
        HIPCHK(m, hipMemcpy(b.kc + hb * KR, k.data(), k.size(), hipMemcpyHostToDevice));
        HIPCHK(m, hipMemcpy(b.ks + hb * NG, s1.data(), s1.size() * 2, hipMemcpyHostToDevice));
        HIPCHK(m, hipMemcpy(b.vs + hb * NG, s2.data(), s2.size() * 2, hipMemcpyHostToDevice));
        HIPCHK(m, hipMemcpy(b.vc + hb * VW, v.data(), v.size() * 4, hipMemcpyHostToDevice));
    }
    return AW4_OK;
}

// Recent-window ring of an attention layer in the logical layout [W][nkv][d]
// (fp16 bits, position t at slot t % W); the library keeps [nkv][W][d].
static int win_copy(aw4_model* m, int32_t layer, uint16_t* kw, uint16_t* vw, bool to_host) {
    if (check_model(m) || !kw || !vw) return AW4_E_INVAL;
    const aw4_config* c = &m->cfg;
    if (layer < 0 || layer >= c->n_layers || m->L[layer].type != 'A' || !m->L[layer].kw)
        return fail(m, AW4_E_INVAL, "not an attention layer with a recent window");
    const int nkv = c->attn_kv_heads, d = c->attn_head_dim, W = c->kv_window;
    LayerBufs& b = m->L[layer];
    HIPCHK(m, hipStreamSynchronize(m->stream));
    std::vector<uint16_t> hk((size_t)nkv * W * d), hv(hk.size());
    if (to_host) {
        HIPCHK(m, hipMemcpy(hk.data(), b.kw, hk.size() * 2, hipMemcpyDeviceToHost));
        HIPCHK(m, hipMemcpy(hv.data(), b.vw, hv.size() * 2, hipMemcpyDeviceToHost));
    }
    for (int w = 0; w < W; ++w)
        for (int j = 0; j < nkv; ++j) {
            uint16_t* lk = kw + ((int64_t)w * nkv + j) * d;
            uint16_t* lv = vw + ((int64_t)w * nkv + j) * d;
            uint16_t* gk = hk.data() + ((int64_t)j * W + w) * d;
            uint16_t* gv = hv.data() + ((int64_t)j * W + w) * d;
            if (to_host) {
                memcpy(lk, gk, (size_t)d * 2);
                memcpy(lv, gv, (size_t)d * 2);
            } else {
                memcpy(gk, lk, (size_t)d * 2);
                memcpy(gv, lv, (size_t)d * 2);
            }
        }
    if (!to_host) {
        HIPCHK(m, hipMemcpy(b.kw, hk.data(), hk.size() * 2, hipMemcpyHostToDevice));
        HIPCHK(m, hipMemcpy(b.vw, hv.data(), hv.size() * 2, hipMemcpyHostToDevice));
    }
    return AW4_OK;
}

int aw4_export_state_win(aw4_model* m, int32_t layer, uint16_t* host_kw, uint16_t* host_vw) {
    return win_copy(m, layer, host_kw, host_vw, true);
}

int aw4_import_state_win(aw4_model* m, int32_t layer, const uint16_t* host_kw, const uint16_t* host_vw) {
    int rc = win_copy(m, layer, const_cast<uint16_t*>(host_kw), const_cast<uint16_t*>(host_vw), false);
    if (rc == AW4_OK) {
        m->win_fresh[(size_t)layer] = true;
        m->win_imported[(size_t)layer] = true;
    }
    return rc;
}

}  // extern "C"

/*
 * CPU oracle for the batch-1 decode step of the hybrid Gated DeltaNet /
 * gated-attention stack with 4-bit weights.  TEST INFRASTRUCTURE ONLY: the
 * tests, the smoke check and the benchmark's CPU-baseline leg may call it;
 * the product library never does, and the two share no code.
 *
 * What it computes follows the reference pages, with the plainest reading
 * taken where they are silent (stated where each applies):
 *  - dense decode, every token runs every layer (page 1, dcwnkz.com estimate,
 *    opening section; page 3 "Qwen3.8-27B 實測", section "部署前必知");
 *  - 48 Gated DeltaNet + 16 full-attention layers (page 3, "部署前必知";
 *    page 5, bs178.com llamAmpere article, "为什么它真能这么快" point 一);
 *  - 4-bit weights (page 1, the "27B x 4 bit" estimate; page 4, jdon.com,
 *    section on quantisation schools, W4A16);
 *  - KV cache with 8-bit keys and rotated ~3-bit values (page 5, point 三);
 *  - a built-in draft head whose output projection covers only a mapped subset
 *    of the vocabulary (page 5, point 四); its block structure is a reading.
 * Formats (group 32, fp16 scales, round-to-nearest-even) follow the readings.
 *
 * Precision: every continuous quantity is computed in fp64.  Where the method
 * fixes a storage format the oracle applies it: GEMV inputs are fp16 (A16),
 * codes and scales of weights and cache are integers and fp16.  Quantisation
 * decisions are taken in fp32, the precision the GPU kernels take them in.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------ fp16 (IEEE 754 binary16) */

/* fp32 -> binary16, round to nearest, ties to even */
uint16_t or_f32_to_f16(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t ax = x & 0x7FFFFFFFu;
    if (ax >= 0x7F800000u) return (uint16_t)(sign | 0x7C00u | (ax > 0x7F800000u ? 0x200u : 0u));
    if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u); /* >= 65520 rounds to inf */
    if (ax < 0x38800000u) {                                   /* below 2^-14: subnormal result */
        float a;
        memcpy(&a, &ax, 4);
        float m = rintf(a * 16777216.0f);                      /* units of 2^-24, exact scaling */
        return (uint16_t)(sign | (uint32_t)m);
    }
    uint32_t e = (ax >> 23) - 127u + 15u;
    uint32_t m = ax & 0x7FFFFFu;
    uint32_t h = (e << 10) | (m >> 13);
    uint32_t rem = m & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h++;
    return (uint16_t)(sign | h);
}

double or_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), e - 25);
    return sign ? -v : v;
}

/* round an fp64 activation to the fp16 GEMV input format (via the fp32 value) */
static inline double to_a16(double v) { return or_f16_to_f64(or_f32_to_f16((float)v)); }

/* ------------------------------------------------------------ codec */

/* Symmetric round-to-nearest group codec: s = fp16(amax / qmax) with the
 * quotient in fp32; c = clamp(rint(x / s), -qmax, qmax); s == 0 gives c = 0. */
void or_quant_group(const float* x, int n, int qmax, uint16_t* s_bits, int8_t* codes) {
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    uint16_t sb = or_f32_to_f16(amax / (float)qmax);
    float s = (float)or_f16_to_f64(sb);
    *s_bits = sb;
    for (int i = 0; i < n; ++i) {
        if (s == 0.0f) { codes[i] = 0; continue; }
        float c = rintf(x[i] / s);
        if (c > (float)qmax) c = (float)qmax;
        if (c < -(float)qmax) c = -(float)qmax;
        codes[i] = (int8_t)c;
    }
}

/* Lloyd-Max 3-bit codebook for a unit-variance Gaussian (J. Max, "Quantizing
 * for minimum distortion", IRE Trans. Inf. Theory, 1960, table for N = 8):
 * output levels +-0.2451, +-0.7560, +-1.3440, +-2.1520, here rounded to fp16.
 * Randomly rotated coordinates of a vector are close to Gaussian, which is
 * why a rotated value cache can use it.  Code c in 0..7 indexes the ascending
 * levels (c < 4 negative). */
static const double kLmMax[4] = {0.2451, 0.7560, 1.3440, 2.1520};

double or_lm_level(int c) {
    if (c < 0 || c > 7) return NAN;
    const double mag = or_f16_to_f64(or_f32_to_f16((float)kLmMax[c < 4 ? 3 - c : c - 4]));
    return c < 4 ? -mag : mag;
}

/* Group codec with the Lloyd-Max codebook: s = fp16(sqrt(mean of x^2)) (the
 * mean square rounded to fp32), t = x / s in fp32, c = the nearest level to t
 * (the number of midpoints between consecutive levels that t exceeds: a tie
 * goes to the lower level); s == 0 gives c = 4 (level +0.2451 times 0). */
void or_quant_group_lm(const float* x, int n, uint16_t* s_bits, int8_t* codes) {
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += (double)x[i] * (double)x[i];
    const uint16_t sb = or_f32_to_f16(sqrtf((float)(ss / n)));
    const float s = (float)or_f16_to_f64(sb);
    *s_bits = sb;
    float mid[7];
    for (int i = 0; i < 7; ++i) mid[i] = (float)(0.5 * (or_lm_level(i) + or_lm_level(i + 1)));
    for (int i = 0; i < n; ++i) {
        if (s == 0.0f) { codes[i] = 4; continue; }
        const float t = x[i] / s;
        int c = 0;
        for (int j = 0; j < 7; ++j) c += t > mid[j];
        codes[i] = (int8_t)c;
    }
}

/* value of one cached V code in format fmt (before the scale) */
static inline double v_level(int fmt, int8_t c) { return fmt == 2 ? or_lm_level(c) : (double)c; }

/* W4 logical format: per row K/2 bytes, element k in the low nibble of byte
 * k/2 when k is even and the high nibble when odd, nibble = code + 8; scales
 * fp16 [rows][K/32]. */
void or_quant_w4_rows(const float* w, int64_t rows, int64_t cols, uint8_t* codes, uint16_t* scales) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        int8_t c[32];
        for (int64_t g = 0; g < cols / 32; ++g) {
            or_quant_group(w + r * cols + g * 32, 32, 7, &scales[r * (cols / 32) + g], c);
            uint8_t* dst = codes + r * (cols / 2) + g * 16;
            for (int i = 0; i < 16; ++i)
                dst[i] = (uint8_t)(((c[2 * i] + 8) & 15) | (((c[2 * i + 1] + 8) & 15) << 4));
        }
    }
}

/* int8 logical format: codes int8 [rows][K], scales fp16 [rows][K/32] */
void or_quant_i8_rows(const float* w, int64_t rows, int64_t cols, int8_t* codes, uint16_t* scales) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t g = 0; g < cols / 32; ++g)
            or_quant_group(w + r * cols + g * 32, 32, 127, &scales[r * (cols / 32) + g],
                           codes + r * cols + g * 32);
}

/* ------------------------------------------------------------ randomized Hadamard transform */

/* Sylvester Hadamard entry: H[i][j] = (-1)^popcount(i & j) */
static inline double had(int i, int j) { return (__builtin_popcount((unsigned)(i & j)) & 1) ? -1.0 : 1.0; }

/* forward: out = H D v / sqrt(d) */
void or_rht_forward(const double* v, const int8_t* signs, int d, double* out) {
    double inv = 1.0 / sqrt((double)d);
    for (int i = 0; i < d; ++i) {
        double a = 0;
        for (int j = 0; j < d; ++j) a += had(i, j) * signs[j] * v[j];
        out[i] = a * inv;
    }
}

/* inverse: out = D H v / sqrt(d)   (H symmetric, H H = d I, D D = I) */
void or_rht_inverse(const double* v, const int8_t* signs, int d, double* out) {
    double inv = 1.0 / sqrt((double)d);
    for (int i = 0; i < d; ++i) {
        double a = 0;
        for (int j = 0; j < d; ++j) a += had(i, j) * v[j];
        out[i] = signs[i] * a * inv;
    }
}

/* ------------------------------------------------------------ model */

typedef struct {
    int32_t hidden, ffn, vocab, n_layers;
    int32_t gdn_qk_heads, gdn_v_heads, gdn_head_dim;
    int32_t attn_q_heads, attn_kv_heads, attn_head_dim;
    int32_t group, max_ctx;
    double rms_eps;
    char pattern[128];
    int32_t draft_vocab;    /* rows of the draft head's vocabulary map, 0 = no draft head */
    int32_t kv_window;      /* recent positions kept at fp16 in the target's caches, 0 = none */
    int32_t kv_format;      /* 0: K int8, V rotated 3-bit uniform; 1: q4_0, K and V 4-bit, V not
                               rotated; 2: K int8, V rotated 3-bit Lloyd-Max codebook */
} or_cfg;

typedef struct { int64_t rows, cols; uint8_t* codes; uint16_t* scales; } or_w4;
typedef struct { int64_t rows, cols; int8_t* codes; uint16_t* scales; } or_i8;

typedef struct {
    char type;
    or_w4 w[5];             /* mixer in, mixer out, ffn gate, ffn up, ffn down */
    double* norm_mix;
    double* norm_ffn;
    double* norm_gated;     /* G */
    double* a_bias;         /* G */
    double* S;              /* G: [nv][dv][dk] */
    int8_t* kc;             /* A: [max_ctx][nkv][dh] */
    uint16_t* ks;           /* A: [max_ctx][nkv][dh/32] */
    int8_t* vc;             /* A: rotated-domain codes in -3..3 */
    uint16_t* vs;
    float* klast;           /* A: fp32 keys of the last appended position [nkv][dh] */
    float* vlast;           /* A: fp32 rotated values of the last appended position */
    int32_t win;            /* A: recent window W (0: every position from the codes) */
    uint16_t* kw;           /* A, W > 0: fp16 keys of the last W positions, slot t % W [W][nkv][dh] */
    uint16_t* vw;           /* A, W > 0: fp16 rotated values, same slots */
} or_layer;

typedef struct {
    or_cfg c;
    or_layer* L;
    or_i8 lm;
    double* norm_final;
    int8_t* signs;
    int32_t pos;
    /* draft head (draft_vocab > 0): fuse [H][2H] over [norm(embedding); norm(hidden)],
     * one gated-attention layer with its own cache of dpos entries, a final norm and
     * the int8 table rows listed in dmap (ascending ids) */
    or_layer D;
    or_w4 fuse;
    double* dn_emb;
    double* dn_hid;
    double* dn_out;
    int32_t* dmap;
    int32_t dpos;
} or_model;

static void* zalloc(size_t n) {
    void* p = calloc(n ? n : 1, 1);
    return p;
}

static int64_t mix_in_rows(const or_cfg* c, char t) {
    if (t == 'G')
        return 2LL * c->gdn_qk_heads * c->gdn_head_dim + 2LL * c->gdn_v_heads * c->gdn_head_dim +
               2LL * c->gdn_v_heads;
    return 2LL * c->attn_q_heads * c->attn_head_dim + 2LL * c->attn_kv_heads * c->attn_head_dim;
}

static int64_t mix_out_cols(const or_cfg* c, char t) {
    return t == 'G' ? (int64_t)c->gdn_v_heads * c->gdn_head_dim : (int64_t)c->attn_q_heads * c->attn_head_dim;
}

static void w4_alloc(or_w4* w, int64_t rows, int64_t cols) {
    w->rows = rows;
    w->cols = cols;
    w->codes = (uint8_t*)zalloc((size_t)(rows * cols / 2));
    w->scales = (uint16_t*)zalloc((size_t)(rows * (cols / 32) * 2));
}

static void layer_alloc(const or_cfg* c, or_layer* L, char type, int32_t win) {
    int64_t H = c->hidden;
    {
        L->type = type;
        w4_alloc(&L->w[0], mix_in_rows(c, L->type), H);
        w4_alloc(&L->w[1], H, mix_out_cols(c, L->type));
        w4_alloc(&L->w[2], c->ffn, H);
        w4_alloc(&L->w[3], c->ffn, H);
        w4_alloc(&L->w[4], H, c->ffn);
        L->norm_mix = (double*)zalloc(sizeof(double) * H);
        L->norm_ffn = (double*)zalloc(sizeof(double) * H);
        if (L->type == 'G') {
            int64_t nv = c->gdn_v_heads, d = c->gdn_head_dim;
            L->norm_gated = (double*)zalloc(sizeof(double) * d);
            L->a_bias = (double*)zalloc(sizeof(double) * nv);
            L->S = (double*)zalloc(sizeof(double) * nv * d * d);
        } else {
            int64_t n = (int64_t)c->max_ctx * c->attn_kv_heads * c->attn_head_dim;
            L->kc = (int8_t*)zalloc(n);
            L->vc = (int8_t*)zalloc(n);
            L->ks = (uint16_t*)zalloc(n / 32 * 2);
            L->vs = (uint16_t*)zalloc(n / 32 * 2);
            L->klast = (float*)zalloc(sizeof(float) * c->attn_kv_heads * c->attn_head_dim);
            L->vlast = (float*)zalloc(sizeof(float) * c->attn_kv_heads * c->attn_head_dim);
            L->win = win;
            if (win > 0) {
                int64_t nw = (int64_t)win * c->attn_kv_heads * c->attn_head_dim;
                L->kw = (uint16_t*)zalloc(nw * 2);
                L->vw = (uint16_t*)zalloc(nw * 2);
            }
        }
    }
}

static void layer_free(or_layer* L) {
    for (int i = 0; i < 5; ++i) { free(L->w[i].codes); free(L->w[i].scales); }
    free(L->norm_mix); free(L->norm_ffn); free(L->norm_gated); free(L->a_bias); free(L->S);
    free(L->kc); free(L->ks); free(L->vc); free(L->vs); free(L->klast); free(L->vlast);
    free(L->kw); free(L->vw);
}

or_model* or_create(const or_cfg* cfg) {
    or_model* m = (or_model*)zalloc(sizeof(or_model));
    m->c = *cfg;
    const or_cfg* c = &m->c;
    int64_t H = c->hidden;
    /* the 4-bit and codebook cache formats serve the single-sequence decode
     * step: no recent window and no draft head with them */
    if (c->draft_vocab < 0 || (c->draft_vocab > 0 && (c->vocab <= 0 || c->draft_vocab > c->vocab)) ||
        c->kv_window < 0 || c->kv_format < 0 || c->kv_format > 2 ||
        (c->kv_format != 0 && (c->kv_window > 0 || c->draft_vocab > 0))) {
        free(m);
        return NULL;
    }
    m->L = (or_layer*)zalloc(sizeof(or_layer) * (size_t)c->n_layers);
    for (int l = 0; l < c->n_layers; ++l) layer_alloc(c, &m->L[l], c->pattern[l], c->kv_window);
    if (c->draft_vocab > 0) {
        layer_alloc(c, &m->D, 'A', 0);   /* the draft head's cache keeps no fp16 window */
        w4_alloc(&m->fuse, H, 2 * H);
        m->dn_emb = (double*)zalloc(sizeof(double) * H);
        m->dn_hid = (double*)zalloc(sizeof(double) * H);
        m->dn_out = (double*)zalloc(sizeof(double) * H);
        m->dmap = (int32_t*)zalloc(sizeof(int32_t) * (size_t)c->draft_vocab);
        for (int32_t i = 0; i < c->draft_vocab; ++i) m->dmap[i] = i;
    }
    if (c->vocab > 0) {
        m->lm.rows = c->vocab;
        m->lm.cols = H;
        m->lm.codes = (int8_t*)zalloc((size_t)c->vocab * H);
        m->lm.scales = (uint16_t*)zalloc((size_t)c->vocab * (H / 32) * 2);
        m->norm_final = (double*)zalloc(sizeof(double) * H);
    }
    m->signs = (int8_t*)zalloc(c->attn_head_dim > 0 ? c->attn_head_dim : 1);
    return m;
}

void or_destroy(or_model* m) {
    if (!m) return;
    for (int l = 0; l < m->c.n_layers; ++l) layer_free(&m->L[l]);
    free(m->L);
    if (m->c.draft_vocab > 0) {
        layer_free(&m->D);
        free(m->fuse.codes); free(m->fuse.scales);
        free(m->dn_emb); free(m->dn_hid); free(m->dn_out); free(m->dmap);
    }
    free(m->lm.codes); free(m->lm.scales); free(m->norm_final); free(m->signs);
    free(m);
}

/* tensor kinds: 0 mixer in, 1 mixer out, 2 ffn gate, 3 ffn up, 4 ffn down (W4);
 * 5 lm_head (int8); 6 mixer norm, 7 ffn norm, 8 gated norm, 9 a bias,
 * 10 final norm (vectors); 11 rotation signs.  Layer n_layers is the draft
 * head's gated-attention layer (kinds 0-4, 6, 7) and holds its fuse matrix
 * (12, W4 [hidden][2 hidden]) and its norms of the embedding (13), of the
 * hidden state (14) and of the output (15). */
static or_layer* layer_ref(or_model* m, int layer) {
    if (layer >= 0 && layer < m->c.n_layers) return &m->L[layer];
    if (layer == m->c.n_layers && m->c.draft_vocab > 0) return &m->D;
    return NULL;
}

static or_w4* w4_ref(or_model* m, int layer, int kind) {
    if (kind == 12) return layer == m->c.n_layers && m->c.draft_vocab > 0 ? &m->fuse : NULL;
    or_layer* L = layer_ref(m, layer);
    if (!L || kind < 0 || kind > 4) return NULL;
    return &L->w[kind];
}

int or_load_w4(or_model* m, int layer, int kind, const uint8_t* codes, const uint16_t* scales) {
    or_w4* w = w4_ref(m, layer, kind);
    if (!w) return -1;
    memcpy(w->codes, codes, (size_t)(w->rows * w->cols / 2));
    memcpy(w->scales, scales, (size_t)(w->rows * (w->cols / 32) * 2));
    return 0;
}

/* quantise fp32 rows [row0, row0+nrows) of a W4 tensor straight into the model */
int or_quant_w4_into(or_model* m, int layer, int kind, int64_t row0, int64_t nrows, const float* w) {
    or_w4* W = w4_ref(m, layer, kind);
    if (!W) return -1;
    if (row0 < 0 || row0 + nrows > W->rows) return -1;
    or_quant_w4_rows(w, nrows, W->cols, W->codes + row0 * (W->cols / 2), W->scales + row0 * (W->cols / 32));
    return 0;
}

int or_quant_lm_into(or_model* m, int64_t row0, int64_t nrows, const float* w) {
    if (m->c.vocab <= 0 || row0 < 0 || row0 + nrows > m->lm.rows) return -1;
    or_quant_i8_rows(w, nrows, m->lm.cols, m->lm.codes + row0 * m->lm.cols,
                     m->lm.scales + row0 * (m->lm.cols / 32));
    return 0;
}

int or_load_i8(or_model* m, const int8_t* codes, const uint16_t* scales) {
    if (m->c.vocab <= 0) return -1;
    memcpy(m->lm.codes, codes, (size_t)(m->lm.rows * m->lm.cols));
    memcpy(m->lm.scales, scales, (size_t)(m->lm.rows * (m->lm.cols / 32) * 2));
    return 0;
}

int or_load_vec(or_model* m, int layer, int kind, const float* v, int n) {
    double* dst = NULL;
    int want = 0;
    if (kind == 10) { dst = m->norm_final; want = m->c.hidden; }
    else if (kind >= 13 && kind <= 15) {
        if (layer != m->c.n_layers || m->c.draft_vocab <= 0) return -1;
        dst = kind == 13 ? m->dn_emb : kind == 14 ? m->dn_hid : m->dn_out;
        want = m->c.hidden;
    } else {
        or_layer* L = layer_ref(m, layer);
        if (!L) return -1;
        if (kind == 6) { dst = L->norm_mix; want = m->c.hidden; }
        if (kind == 7) { dst = L->norm_ffn; want = m->c.hidden; }
        if (kind == 8) { dst = L->norm_gated; want = m->c.gdn_head_dim; }
        if (kind == 9) { dst = L->a_bias; want = m->c.gdn_v_heads; }
    }
    if (!dst || n != want) return -1;
    for (int i = 0; i < n; ++i) dst[i] = (double)v[i];
    return 0;
}

int or_load_signs(or_model* m, const int8_t* s, int n) {
    if (n != m->c.attn_head_dim) return -1;
    memcpy(m->signs, s, (size_t)n);
    return 0;
}

/* ------------------------------------------------------------ building blocks */

static void gemv_w4(const or_w4* W, const double* x, double* y) {
    int64_t K = W->cols, G = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < W->rows; ++n) {
        const uint8_t* c = W->codes + n * (K / 2);
        const uint16_t* s = W->scales + n * G;
        double acc = 0.0;
        for (int64_t g = 0; g < G; ++g) {
            double sc = or_f16_to_f64(s[g]);
            for (int64_t k = 32 * g; k < 32 * g + 32; ++k) {
                int nib = (k & 1) ? (c[k >> 1] >> 4) : (c[k >> 1] & 15);
                acc += ((double)(nib - 8) * sc) * x[k];
            }
        }
        y[n] = acc;
    }
}

static void gemv_i8(const or_i8* W, const double* x, double* y) {
    int64_t K = W->cols, G = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < W->rows; ++n) {
        const int8_t* c = W->codes + n * K;
        const uint16_t* s = W->scales + n * G;
        double acc = 0.0;
        for (int64_t g = 0; g < G; ++g) {
            double sc = or_f16_to_f64(s[g]);
            for (int64_t k = 32 * g; k < 32 * g + 32; ++k) acc += ((double)c[k] * sc) * x[k];
        }
        y[n] = acc;
    }
}

/* RMSNorm: out = x / sqrt(mean(x^2) + eps) * w, rounded to the fp16 input format */
static void rmsnorm_a16(const double* x, const double* w, int64_t n, double eps, double* out) {
    double ss = 0;
    for (int64_t i = 0; i < n; ++i) ss += x[i] * x[i];
    double r = 1.0 / sqrt(ss / (double)n + eps);
    for (int64_t i = 0; i < n; ++i) out[i] = to_a16(x[i] * r * w[i]);
}

static inline double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }
static inline double silu(double v) { return v * sigmoid(v); }

/* One Gated DeltaNet head step, expanded form of
 *   S <- alpha * S (I - beta k k^T) + beta v k^T ,   o = S q
 * i.e. S <- alpha * (S - beta (S k) k^T) + beta v k^T.  S is [dv][dk] row-major. */
void or_gdn_head_step(double* S, const double* k, const double* v, const double* q, double alpha,
                      double beta, int dv, int dk, double* o) {
    for (int i = 0; i < dv; ++i) {
        double* row = S + (int64_t)i * dk;
        double u = 0;
        for (int j = 0; j < dk; ++j) u += row[j] * k[j];
        double oi = 0;
        for (int j = 0; j < dk; ++j) {
            row[j] = alpha * (row[j] - beta * u * k[j]) + beta * v[i] * k[j];
            oi += row[j] * q[j];
        }
        o[i] = oi;
    }
}

static void l2norm(const double* x, int n, double eps, double* out) {
    double ss = 0;
    for (int i = 0; i < n; ++i) ss += x[i] * x[i];
    double r = 1.0 / sqrt(ss + eps);
    for (int i = 0; i < n; ++i) out[i] = x[i] * r;
}

static void gdn_mixer(or_model* m, or_layer* L, const double* xh, double* delta) {
    const or_cfg* c = &m->c;
    int nqk = c->gdn_qk_heads, nv = c->gdn_v_heads, d = c->gdn_head_dim;
    int64_t rows = L->w[0].rows;
    double* p = (double*)malloc(sizeof(double) * rows);
    gemv_w4(&L->w[0], xh, p);
    double* q = p;
    double* k = q + (int64_t)nqk * d;
    double* v = k + (int64_t)nqk * d;
    double* z = v + (int64_t)nv * d;
    double* a = z + (int64_t)nv * d;
    double* b = a + nv;
    double* qn = (double*)malloc(sizeof(double) * nqk * d);
    double* kn = (double*)malloc(sizeof(double) * nqk * d);
    for (int j = 0; j < nqk; ++j) {
        l2norm(q + (int64_t)j * d, d, c->rms_eps, qn + (int64_t)j * d);
        l2norm(k + (int64_t)j * d, d, c->rms_eps, kn + (int64_t)j * d);
    }
    double* y = (double*)malloc(sizeof(double) * nv * d);
    double* o = (double*)malloc(sizeof(double) * d);
    int ratio = nv / nqk;
    for (int h = 0; h < nv; ++h) {
        int j = h / ratio;
        double alpha = sigmoid(a[h] + L->a_bias[h]);
        double beta = sigmoid(b[h]);
        or_gdn_head_step(L->S + (int64_t)h * d * d, kn + (int64_t)j * d, v + (int64_t)h * d,
                         qn + (int64_t)j * d, alpha, beta, d, d, o);
        /* gated RMSNorm: RMSNorm(o) * w * SiLU(z) */
        double ss = 0;
        for (int i = 0; i < d; ++i) ss += o[i] * o[i];
        double r = 1.0 / sqrt(ss / d + c->rms_eps);
        for (int i = 0; i < d; ++i)
            y[(int64_t)h * d + i] = to_a16(o[i] * r * L->norm_gated[i] * silu(z[(int64_t)h * d + i]));
    }
    gemv_w4(&L->w[1], y, delta);
    free(p); free(qn); free(kn); free(y); free(o);
}

/* One query head over npos cached positions (stride = elements between
 * consecutive positions of this kv head):
 *   s_t = q . K~_t / sqrt(d),  p = softmax(s),  acc = sum_t p_t V~'_t,
 *   out = RHT^-1(acc)   (values are cached in the rotated domain).
 * K~_t, V~'_t are the dequantised codes, except for the last `win` positions
 * (win > 0), which are read at fp16 from the window ring kw/vw (position t at
 * slot t % win, slots wstride elements apart).  The recent-window variant of
 * the KV cache: page 3 (Qwen3.8-27B 實測), section "RTX 4090 24GB", whose
 * 130K configuration keeps the last 2,048 tokens at F16 against attention
 * drift while older positions stay quantised. */
void or_attend_head_fmt(const double* q, const int8_t* kc, const uint16_t* ks, const int8_t* vc,
                        const uint16_t* vs, int64_t npos, int64_t stride, int d, const int8_t* signs,
                        const uint16_t* kw, const uint16_t* vw, int64_t win, int64_t wstride, int fmt,
                        double* out) {
    double* s = (double*)malloc(sizeof(double) * (npos > 0 ? npos : 1));
    double* acc = (double*)calloc(d, sizeof(double));
    double scale = 1.0 / sqrt((double)d);
    double mx = -INFINITY;
    const int64_t w0 = win > 0 ? npos - win : npos;   /* first position read from the window */
    for (int64_t t = 0; t < npos; ++t) {
        double dot = 0;
        if (t >= w0) {
            const uint16_t* kr = kw + (t % win) * wstride;
            for (int e = 0; e < d; ++e) dot += q[e] * or_f16_to_f64(kr[e]);
        } else {
            const int8_t* kr = kc + t * stride;
            const uint16_t* kq = ks + t * stride / 32;
            for (int e = 0; e < d; ++e) dot += q[e] * ((double)kr[e] * or_f16_to_f64(kq[e / 32]));
        }
        s[t] = dot * scale;
        if (s[t] > mx) mx = s[t];
    }
    double sum = 0;
    for (int64_t t = 0; t < npos; ++t) { s[t] = exp(s[t] - mx); sum += s[t]; }
    for (int64_t t = 0; t < npos; ++t) {
        double pt = s[t] / sum;
        if (t >= w0) {
            const uint16_t* vr = vw + (t % win) * wstride;
            for (int e = 0; e < d; ++e) acc[e] += pt * or_f16_to_f64(vr[e]);
        } else {
            const int8_t* vr = vc + t * stride;
            const uint16_t* vq = vs + t * stride / 32;
            for (int e = 0; e < d; ++e) acc[e] += pt * (v_level(fmt, vr[e]) * or_f16_to_f64(vq[e / 32]));
        }
    }
    /* formats 0 and 2 cache rotated values: undo the rotation once */
    if (fmt == 1) memcpy(out, acc, sizeof(double) * d);
    else or_rht_inverse(acc, signs, d, out);
    free(s);
    free(acc);
}

void or_attend_head(const double* q, const int8_t* kc, const uint16_t* ks, const int8_t* vc,
                    const uint16_t* vs, int64_t npos, int64_t stride, int d, const int8_t* signs,
                    const uint16_t* kw, const uint16_t* vw, int64_t win, int64_t wstride, double* out) {
    or_attend_head_fmt(q, kc, ks, vc, vs, npos, stride, d, signs, kw, vw, win, wstride, 0, out);
}

/* K and V of one kv head into the cache at one position, decisions taken in
 * fp32.  Format 0: K int8 per 32 of the fp32 key; V rotated (RHT) then 3-bit
 * per 32.  Format 1 (q4_0, page 3 "Qwen3.8-27B 實測" and page 4, jdon.com:
 * both caches at 4 bits for long contexts on small cards): K and V each 4-bit
 * per 32 with an fp16 scale (the W4 codec), V not rotated.  Format 2: K int8;
 * V rotated, then the Lloyd-Max codebook per 32. */
void or_kv_encode_fmt(const double* k, const double* v, const int8_t* signs, int d, int fmt, int8_t* kc,
                      uint16_t* ks, int8_t* vc, uint16_t* vs) {
    float* tmp = (float*)malloc(sizeof(float) * d);
    double* vr = (double*)malloc(sizeof(double) * d);
    for (int i = 0; i < d; ++i) tmp[i] = (float)k[i];
    for (int gi = 0; gi < d / 32; ++gi) or_quant_group(tmp + gi * 32, 32, fmt == 1 ? 7 : 127, &ks[gi], kc + gi * 32);
    if (fmt == 1) memcpy(vr, v, sizeof(double) * d);
    else or_rht_forward(v, signs, d, vr);
    for (int i = 0; i < d; ++i) tmp[i] = (float)vr[i];
    for (int gi = 0; gi < d / 32; ++gi) {
        if (fmt == 2) or_quant_group_lm(tmp + gi * 32, 32, &vs[gi], vc + gi * 32);
        else or_quant_group(tmp + gi * 32, 32, fmt == 1 ? 7 : 3, &vs[gi], vc + gi * 32);
    }
    free(tmp);
    free(vr);
}

void or_kv_encode(const double* k, const double* v, const int8_t* signs, int d, int8_t* kc, uint16_t* ks,
                  int8_t* vc, uint16_t* vs) {
    or_kv_encode_fmt(k, v, signs, d, 0, kc, ks, vc, vs);
}

/* the fp32 key and (rotated, except in format 1) value the last append
 * quantised (for tie checks) */
static void kv_record(const double* k, const double* v, const int8_t* signs, int d, int fmt, float* kl,
                      float* vl) {
    double* vr = (double*)malloc(sizeof(double) * d);
    for (int i = 0; i < d; ++i) kl[i] = (float)k[i];
    if (fmt == 1) memcpy(vr, v, sizeof(double) * d);
    else or_rht_forward(v, signs, d, vr);
    for (int i = 0; i < d; ++i) vl[i] = (float)vr[i];
    free(vr);
}

/* gated attention: append the token at cache entry t, attend over entries 0..t,
 * gate each head output by sigmoid(g), project back */
static void attn_mixer(or_model* m, or_layer* L, int64_t t, const double* xh, double* delta) {
    const or_cfg* c = &m->c;
    int nq = c->attn_q_heads, nkv = c->attn_kv_heads, d = c->attn_head_dim;
    int64_t rows = L->w[0].rows;
    double* p = (double*)malloc(sizeof(double) * rows);
    gemv_w4(&L->w[0], xh, p);
    double* q = p;
    double* g = q + (int64_t)nq * d;
    double* k = g + (int64_t)nq * d;
    double* v = k + (int64_t)nkv * d;
    for (int j = 0; j < nkv; ++j) {
        int64_t base = (t * nkv + j) * d;
        or_kv_encode_fmt(k + (int64_t)j * d, v + (int64_t)j * d, m->signs, d, c->kv_format, L->kc + base,
                         L->ks + base / 32, L->vc + base, L->vs + base / 32);
        kv_record(k + (int64_t)j * d, v + (int64_t)j * d, m->signs, d, c->kv_format, L->klast + (int64_t)j * d,
                  L->vlast + (int64_t)j * d);
        if (L->win > 0) {
            /* the window keeps the fp32 key and rotated value rounded to fp16 */
            int64_t slot = ((t % L->win) * nkv + j) * d;
            for (int e = 0; e < d; ++e) {
                L->kw[slot + e] = or_f32_to_f16(L->klast[(int64_t)j * d + e]);
                L->vw[slot + e] = or_f32_to_f16(L->vlast[(int64_t)j * d + e]);
            }
        }
    }
    double* o = (double*)malloc(sizeof(double) * nq * d);
    int ratio = nq / nkv;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < nq; ++i) {
        int j = i / ratio;
        int64_t off = (int64_t)j * d;
        or_attend_head_fmt(q + (int64_t)i * d, L->kc + off, L->ks + off / 32, L->vc + off, L->vs + off / 32,
                           t + 1, (int64_t)nkv * d, d, m->signs, L->win > 0 ? L->kw + off : NULL,
                           L->win > 0 ? L->vw + off : NULL, L->win, (int64_t)nkv * d, c->kv_format,
                           o + (int64_t)i * d);
        for (int e = 0; e < d; ++e)
            o[(int64_t)i * d + e] = to_a16(o[(int64_t)i * d + e] * sigmoid(g[(int64_t)i * d + e]));
    }
    gemv_w4(&L->w[1], o, delta);
    free(p);
    free(o);
}

static void ffn(or_model* m, or_layer* L, const double* xh, double* delta) {
    int64_t F = m->c.ffn;
    double* gt = (double*)malloc(sizeof(double) * F);
    double* up = (double*)malloc(sizeof(double) * F);
    gemv_w4(&L->w[2], xh, gt);
    gemv_w4(&L->w[3], xh, up);
    for (int64_t i = 0; i < F; ++i) gt[i] = to_a16(silu(gt[i]) * up[i]);
    gemv_w4(&L->w[4], gt, delta);
    free(gt); free(up);
}

/* Run every layer at the current position on residual x (in place); append
 * the cache entry, update the recurrent states and advance the position.
 * trace (optional) receives the residual after each layer, [n_layers][H]. */
/* one pre-norm residual block: x += mixer(norm(x)); x += ffn(norm(x)); an
 * attention mixer writes cache entry t (xh, dl: scratch of H doubles) */
static void layer_forward(or_model* m, or_layer* L, int64_t t, double* x, double* xh, double* dl) {
    const or_cfg* c = &m->c;
    int64_t H = c->hidden;
    rmsnorm_a16(x, L->norm_mix, H, c->rms_eps, xh);
    if (L->type == 'G') gdn_mixer(m, L, xh, dl);
    else attn_mixer(m, L, t, xh, dl);
    for (int64_t i = 0; i < H; ++i) x[i] += dl[i];
    rmsnorm_a16(x, L->norm_ffn, H, c->rms_eps, xh);
    ffn(m, L, xh, dl);
    for (int64_t i = 0; i < H; ++i) x[i] += dl[i];
}

int or_forward_layers(or_model* m, double* x, double* trace) {
    const or_cfg* c = &m->c;
    if (m->pos >= c->max_ctx) return -2;
    int64_t H = c->hidden;
    double* xh = (double*)malloc(sizeof(double) * H);
    double* dl = (double*)malloc(sizeof(double) * H);
    for (int l = 0; l < c->n_layers; ++l) {
        layer_forward(m, &m->L[l], m->pos, x, xh, dl);
        if (trace) memcpy(trace + (int64_t)l * H, x, sizeof(double) * H);
    }
    m->pos++;
    free(xh); free(dl);
    return 0;
}

/* embedding row of the tied int8 table, dequantised exactly */
int or_embed(or_model* m, int32_t token, double* x) {
    if (m->c.vocab <= 0 || token < 0 || token >= m->c.vocab) return -1;
    int64_t H = m->c.hidden;
    for (int64_t k = 0; k < H; ++k)
        x[k] = (double)m->lm.codes[token * H + k] * or_f16_to_f64(m->lm.scales[token * (H / 32) + k / 32]);
    return 0;
}

/* final RMSNorm + int8 lm_head + argmax (lowest index wins ties) */
int or_head(or_model* m, const double* x, double* logits, int32_t* argmax) {
    if (m->c.vocab <= 0) return -1;
    int64_t H = m->c.hidden;
    double* xh = (double*)malloc(sizeof(double) * H);
    rmsnorm_a16(x, m->norm_final, H, m->c.rms_eps, xh);
    gemv_i8(&m->lm, xh, logits);
    int32_t best = 0;
    for (int32_t i = 1; i < m->c.vocab; ++i)
        if (logits[i] > logits[best]) best = i;
    if (argmax) *argmax = best;
    free(xh);
    return 0;
}

int or_decode_token(or_model* m, int32_t token, double* x_out, double* logits, int32_t* argmax) {
    int64_t H = m->c.hidden;
    double* x = (double*)malloc(sizeof(double) * H);
    int rc = or_embed(m, token, x);
    if (!rc) rc = or_forward_layers(m, x, NULL);
    if (!rc) rc = or_head(m, x, logits, argmax);
    if (!rc && x_out) memcpy(x_out, x, sizeof(double) * H);
    free(x);
    return rc;
}

int32_t or_get_pos(const or_model* m) { return m->pos; }

/* ------------------------------------------------------------ draft head
 * The pages' draft head (page 5, bs178.com llamAmpere article, "为什么它真能这么快"
 * point 四) proposes tokens from the target's last hidden state and scores them
 * with a projection restricted to a list of token ids (the vocabulary map);
 * the target still chooses from the full vocabulary.  Readings: the block
 * combines the normalised embedding of the current token with the normalised
 * hidden state through one W4 matrix, runs one gated-attention layer of the
 * target's shape with its own cache, and scores the normalised result with the
 * tied int8 table rows of the mapped ids. */

static int cmp_i32(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return x < y ? -1 : x > y;
}

/* the map as distinct ids in [0, vocab), stored ascending */
int or_set_draft_map(or_model* m, const int32_t* ids, int32_t n) {
    if (m->c.draft_vocab <= 0 || n != m->c.draft_vocab) return -1;
    int32_t* t = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    memcpy(t, ids, sizeof(int32_t) * (size_t)n);
    qsort(t, (size_t)n, sizeof(int32_t), cmp_i32);
    for (int32_t i = 0; i < n; ++i)
        if (t[i] < 0 || t[i] >= m->c.vocab || (i > 0 && t[i] == t[i - 1])) { free(t); return -1; }
    memcpy(m->dmap, t, sizeof(int32_t) * (size_t)n);
    free(t);
    return 0;
}

int or_get_draft_map(const or_model* m, int32_t* ids) {
    if (m->c.draft_vocab <= 0) return -1;
    memcpy(ids, m->dmap, sizeof(int32_t) * (size_t)m->c.draft_vocab);
    return 0;
}

/* One step of the draft head on (token, h): writes cache entry dpos + slot and
 * attends over entries 0 .. dpos + slot; the entry count dpos is left alone.
 * x_out (optional): the block's output hidden state [H]; logits (optional):
 * the mapped scores [draft_vocab] in ascending-id order. */
int or_draft_step(or_model* m, int32_t token, const double* h, int32_t slot, double* x_out, double* logits) {
    const or_cfg* c = &m->c;
    if (c->draft_vocab <= 0 || token < 0 || token >= c->vocab || slot < 0) return -1;
    int64_t t = (int64_t)m->dpos + slot;
    if (t >= c->max_ctx) return -2;
    int64_t H = c->hidden;
    double* e = (double*)malloc(sizeof(double) * H);
    double* u = (double*)malloc(sizeof(double) * 2 * H);
    double* x = (double*)malloc(sizeof(double) * H);
    double* xh = (double*)malloc(sizeof(double) * H);
    double* dl = (double*)malloc(sizeof(double) * H);
    or_embed(m, token, e);
    rmsnorm_a16(e, m->dn_emb, H, c->rms_eps, u);
    rmsnorm_a16(h, m->dn_hid, H, c->rms_eps, u + H);
    gemv_w4(&m->fuse, u, x);
    layer_forward(m, &m->D, t, x, xh, dl);
    if (x_out) memcpy(x_out, x, sizeof(double) * H);
    if (logits) {
        rmsnorm_a16(x, m->dn_out, H, c->rms_eps, xh);
        int64_t G = H / 32;
#pragma omp parallel for schedule(static)
        for (int32_t i = 0; i < c->draft_vocab; ++i) {
            const int8_t* cr = m->lm.codes + (int64_t)m->dmap[i] * H;
            const uint16_t* sr = m->lm.scales + (int64_t)m->dmap[i] * G;
            double acc = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                double sc = or_f16_to_f64(sr[g]);
                for (int64_t k = 32 * g; k < 32 * g + 32; ++k) acc += ((double)cr[k] * sc) * xh[k];
            }
            logits[i] = acc;
        }
    }
    free(e); free(u); free(x); free(xh); free(dl);
    return 0;
}

int32_t or_get_dpos(const or_model* m) { return m->dpos; }

int or_set_dpos(or_model* m, int32_t dpos) {
    if (m->c.draft_vocab <= 0 || dpos < 0 || dpos > m->c.max_ctx) return -1;
    m->dpos = dpos;
    return 0;
}

/* ------------------------------------------------------------ state import / export
 * Logical state: position; per GDN layer fp32 S [nv][dv][dk]; per attention
 * layer K codes int8 [pos][nkv][dh], K scales fp16 [pos][nkv][dh/32], V codes
 * int8 [pos][nkv][dh] (format 0: -3..3; format 1: -7..7, keys too; format 2:
 * level index 0..7), V scales fp16 [pos][nkv][dh/32]. */
int or_set_state_gdn(or_model* m, int layer, const float* S) {
    if (layer < 0 || layer >= m->c.n_layers || m->L[layer].type != 'G') return -1;
    int64_t n = (int64_t)m->c.gdn_v_heads * m->c.gdn_head_dim * m->c.gdn_head_dim;
    for (int64_t i = 0; i < n; ++i) m->L[layer].S[i] = (double)S[i];
    return 0;
}

/* the state at full precision: a verify pass puts back exactly the state it
 * saved before running the drafts */
int or_set_state_gdn64(or_model* m, int layer, const double* S) {
    if (layer < 0 || layer >= m->c.n_layers || m->L[layer].type != 'G') return -1;
    int64_t n = (int64_t)m->c.gdn_v_heads * m->c.gdn_head_dim * m->c.gdn_head_dim;
    memcpy(m->L[layer].S, S, sizeof(double) * n);
    return 0;
}

int or_get_state_gdn(const or_model* m, int layer, double* S) {
    if (layer < 0 || layer >= m->c.n_layers || m->L[layer].type != 'G') return -1;
    int64_t n = (int64_t)m->c.gdn_v_heads * m->c.gdn_head_dim * m->c.gdn_head_dim;
    memcpy(S, m->L[layer].S, sizeof(double) * n);
    return 0;
}

int or_set_state_kv(or_model* m, int layer, int32_t npos, const int8_t* kc, const uint16_t* ks,
                    const int8_t* vc, const uint16_t* vs) {
    or_layer* L = layer_ref(m, layer);
    if (!L || L->type != 'A') return -1;
    if (npos < 0 || npos > m->c.max_ctx) return -1;
    int64_t n = (int64_t)npos * m->c.attn_kv_heads * m->c.attn_head_dim;
    memcpy(L->kc, kc, n);
    memcpy(L->vc, vc, n);
    memcpy(L->ks, ks, n / 32 * 2);
    memcpy(L->vs, vs, n / 32 * 2);
    return 0;
}

int or_get_state_kv(or_model* m, int layer, int32_t npos, int8_t* kc, uint16_t* ks, int8_t* vc,
                    uint16_t* vs) {
    const or_layer* L = layer_ref(m, layer);
    if (!L || L->type != 'A') return -1;
    if (npos < 0 || npos > m->c.max_ctx) return -1;
    int64_t n = (int64_t)npos * m->c.attn_kv_heads * m->c.attn_head_dim;
    memcpy(kc, L->kc, n);
    memcpy(vc, L->vc, n);
    memcpy(ks, L->ks, n / 32 * 2);
    memcpy(vs, L->vs, n / 32 * 2);
    return 0;
}

/* The fp16 window ring of an attention layer: keys and rotated values of the
 * last W positions, position t at slot t % W, [W][nkv][dh] fp16 bits each. */
int or_set_state_win(or_model* m, int layer, const uint16_t* kw, const uint16_t* vw) {
    if (layer < 0 || layer >= m->c.n_layers || m->L[layer].type != 'A' || m->L[layer].win <= 0) return -1;
    int64_t n = (int64_t)m->L[layer].win * m->c.attn_kv_heads * m->c.attn_head_dim;
    memcpy(m->L[layer].kw, kw, n * 2);
    memcpy(m->L[layer].vw, vw, n * 2);
    return 0;
}

int or_get_state_win(const or_model* m, int layer, uint16_t* kw, uint16_t* vw) {
    if (layer < 0 || layer >= m->c.n_layers || m->L[layer].type != 'A' || m->L[layer].win <= 0) return -1;
    int64_t n = (int64_t)m->L[layer].win * m->c.attn_kv_heads * m->c.attn_head_dim;
    memcpy(kw, m->L[layer].kw, n * 2);
    memcpy(vw, m->L[layer].vw, n * 2);
    return 0;
}

int or_get_last_kv(const or_model* m, int layer, float* k, float* vrot) {
    if (layer < 0 || layer >= m->c.n_layers || m->L[layer].type != 'A') return -1;
    int64_t n = (int64_t)m->c.attn_kv_heads * m->c.attn_head_dim;
    memcpy(k, m->L[layer].klast, sizeof(float) * n);
    memcpy(vrot, m->L[layer].vlast, sizeof(float) * n);
    return 0;
}

int or_set_pos(or_model* m, int32_t pos) {
    if (pos < 0 || pos > m->c.max_ctx) return -1;
    m->pos = pos;
    return 0;
}

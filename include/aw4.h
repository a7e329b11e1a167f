/*
 * aw4.h - C ABI of the MI355X (gfx950) batch-1 decode library for a hybrid
 * Gated DeltaNet / gated-attention language model with 4-bit weights.
 *
 * What the library computes (where the pages are silent, the plainest reading
 * is taken and stated where it applies):
 *  - Decode is bandwidth-bound: every token streams all weights from memory
 *    (page 5, bs178.com llamAmpere article, "为什么它真能这么快" point 二;
 *    page 3 "Qwen3.8-27B 實測", section "部署前必知").
 *  - The stack interleaves Gated DeltaNet recurrent layers with full-attention
 *    layers, 48 + 16 in the 27B model (page 3, "部署前必知"; page 5 point 一).
 *  - Weights are 4-bit (W4A16: 4-bit weights, 16-bit activations; page 4,
 *    jdon.com, section on quantisation schools; page 1, the "27B x 4 bit"
 *    estimate), here symmetric codes in groups of 32 with an fp16 scale; the
 *    output head is int8 and doubles as the embedding table.
 *  - The KV cache stores keys at 8 bits and values rotated and compressed to
 *    about 3 bits (page 5, point 三): keys int8 per 32 with an fp16 scale, values
 *    multiplied by a random-sign Walsh-Hadamard matrix then 3-bit per 32.
 *  - verify_k checks draft tokens with acceptance probability min(1, p/q) and
 *    residual resampling (page 5, point 四).
 *  - The model's own draft head proposes those tokens and scores them only over
 *    a list of token ids, the vocabulary map; the target keeps the full
 *    vocabulary (page 5, point 四).
 *
 * Conventions for every entry point:
 *  - Returns AW4_OK (0) or a negative AW4_E_* code; no exception crosses the
 *    ABI.  aw4_last_error() gives a message for the last failure on a model.
 *  - "dev_" pointers are device (HIP) addresses, "host_" pointers are host
 *    memory.  The library never frees caller memory.
 *  - One model is bound to one device and one HIP stream; calls on one model
 *    must not overlap (not thread-safe).  Host buffers are read or written only
 *    during the call.
 *  - Entry points that only enqueue work return before it finishes; those that
 *    return data on the host synchronise the stream first.
 */
#ifndef AW4_H
#define AW4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AW4_OK 0
#define AW4_E_INVAL (-1)       /* bad argument or unsupported shape */
#define AW4_E_ARENA (-2)       /* arena missing, misaligned or too small */
#define AW4_E_NODEVICE (-3)    /* no HIP device / not gfx950 */
#define AW4_E_HIP (-4)         /* a HIP runtime call failed */
#define AW4_E_FORMAT (-5)      /* weight blob: bad magic, version, size or config echo */
#define AW4_E_CTX_FULL (-6)    /* position would exceed max_ctx */
#define AW4_E_TOKEN (-7)       /* token id outside [0, vocab) */
#define AW4_E_STATE (-8)       /* call not valid in the model's current state */

/* Model shape.  Requirements (else AW4_E_INVAL): hidden, ffn multiples of 64;
 * group == 32; n_layers in [1, 127], layer_pattern holds n_layers letters
 * 'G' (Gated DeltaNet) or 'A' (gated attention); GDN: gdn_head_dim in {64, 128},
 * gdn_v_heads a multiple of gdn_qk_heads; attention: attn_head_dim in {64, 256},
 * attn_q_heads a multiple of attn_kv_heads, attn_q_heads/attn_kv_heads <= 8;
 * vocab in [0, 2097152] (0: no embedding or output head, only aw4_decode_hidden works);
 * max_ctx >= 1; max_verify in [1, 4]; rms_eps > 0; draft_vocab in [0, vocab]
 * (0: no draft head; otherwise the attention fields must describe a valid
 * attention layer even when the pattern holds none, since the draft head's
 * block has that shape, and hidden <= 8192); max_batch in [0, 4];
 * kv_window in [0, max_ctx], and with kv_window > 0 also max_batch <= 1 and
 * draft_vocab == 0.
 *
 * Recent window (kv_window = W > 0; page 3, "Qwen3.8-27B 實測", section
 * "RTX 4090 24GB": a 130K configuration keeps the last 2,048 tokens at F16
 * against attention drift).  Every appended position still gets its int8 key
 * and 3-bit rotated value codes; in addition the fp32 key and the fp32 rotated
 * value are kept rounded to fp16 in a ring of W slots (position t at slot
 * t % W).  A decode step at position p reads positions p - W + 1 .. p from the
 * ring and the older ones from their codes.  Only the single-sequence decode
 * path reads the window: aw4_prefill runs token by token (no chunks),
 * aw4_verify_k and aw4_decode_batch return AW4_E_INVAL.
 *
 * KV-cache codecs (kv_format).  0: keys int8 per 32 with an fp16 scale, values
 * rotated by the random-sign Walsh-Hadamard transform then 3-bit codes -3..3 per
 * 32 (page 5, bs178.com llamAmpere article, "为什么它真能这么快" point 三).
 * 1, q4_0 (page 3, "Qwen3.8-27B 實測", section "RTX 5090 32GB：可以四人", runs
 * 131K with both caches at q4_0; page 4, jdon.com, on fitting 262K into 24 GB):
 * keys and values each 4-bit codes -7..7 per 32 with an fp16 scale (the W4
 * weight codec), values not rotated.  2: keys int8; values rotated, then per 32
 * the index 0..7 of the nearest level of the 8-level Lloyd-Max codebook of a
 * unit Gaussian (J. Max 1960: +-0.2451, +-0.7560, +-1.3440, +-2.1520, as fp16),
 * scaled by fp16 of the group's root mean square, ties to the lower level.
 * Formats 1 and 2 serve the single-sequence decode step: they need kv_window 0,
 * max_batch <= 1 and draft_vocab 0; aw4_prefill runs token by token and
 * aw4_verify_k returns AW4_E_INVAL.  The state calls use the logical codes of
 * the format (format 1: K and V -7..7; format 2: V indices 0..7). */
typedef struct aw4_config {
    int32_t hidden;
    int32_t ffn;
    int32_t vocab;
    int32_t n_layers;
    int32_t gdn_qk_heads;
    int32_t gdn_v_heads;
    int32_t gdn_head_dim;
    int32_t attn_q_heads;
    int32_t attn_kv_heads;
    int32_t attn_head_dim;
    int32_t group;
    int32_t max_ctx;
    int32_t max_verify;
    float rms_eps;
    char layer_pattern[128];
    int32_t draft_vocab;        /* ids in the draft head's vocabulary map */
    int32_t max_batch;          /* sequences with their own state (0 or 1: one; at most 4) */
    int32_t kv_window;          /* recent window: the last kv_window positions of every
                                   attention layer are read at fp16 (0: none); see below */
    int32_t kv_format;          /* KV-cache codecs (0, 1 or 2); see below */
} aw4_config;

typedef struct aw4_model aw4_model;

/* Tensor kinds.  Per-layer W4 matrices [rows x cols], y = W x:
 *   MIX_IN   GDN: rows [q | k | v | z | a | b] = 2*nqk*d + 2*nv*d + 2*nv;
 *            attention: rows [q | g | k | v] = 2*nq*dh + 2*nkv*dh; cols hidden.
 *   MIX_OUT  [hidden x nv*d] (GDN) or [hidden x nq*dh] (attention).
 *   FFN_GATE, FFN_UP [ffn x hidden]; FFN_DOWN [hidden x ffn].
 * Global: LM_HEAD int8 [vocab x hidden] (also the embedding table).
 * Vectors (fp32): NORM_MIX, NORM_FFN [hidden]; NORM_GATED [gdn_head_dim];
 * A_BIAS [gdn_v_heads]; NORM_FINAL [hidden]; RHT_SIGNS [attn_head_dim] (+1/-1).
 * Draft head (draft_vocab > 0), all at layer index n_layers: one gated-attention
 * layer (MIX_IN, MIX_OUT, FFN_*, NORM_MIX, NORM_FFN as above) and
 *   DRAFT_FUSE      W4 [hidden x 2*hidden], x = W [u_e; u_h] with
 *                   u_e = RMSNorm(embedding(t)) * DRAFT_NORM_EMB and
 *                   u_h = RMSNorm(h) * DRAFT_NORM_HID, both in fp16;
 *   DRAFT_NORM_EMB, DRAFT_NORM_HID, DRAFT_NORM_OUT  vectors [hidden];
 *   DRAFT_MAP       int32 ids [draft_vocab] (aw4_set_draft_map). */
enum {
    AW4_T_MIX_IN = 0,
    AW4_T_MIX_OUT = 1,
    AW4_T_FFN_GATE = 2,
    AW4_T_FFN_UP = 3,
    AW4_T_FFN_DOWN = 4,
    AW4_T_LM_HEAD = 5,
    AW4_T_NORM_MIX = 6,
    AW4_T_NORM_FFN = 7,
    AW4_T_NORM_GATED = 8,
    AW4_T_A_BIAS = 9,
    AW4_T_NORM_FINAL = 10,
    AW4_T_RHT_SIGNS = 11,
    AW4_T_DRAFT_FUSE = 12,
    AW4_T_DRAFT_NORM_EMB = 13,
    AW4_T_DRAFT_NORM_HID = 14,
    AW4_T_DRAFT_NORM_OUT = 15,
    AW4_T_DRAFT_MAP = 16
};

/* ----------------------------------------------------------- lifetime */

/* Pure host check of a config; enqueues nothing. */
int aw4_validate_config(const aw4_config* cfg);

/* Bytes of device memory the model needs (weights, caches, states, scratch),
 * written to *out_bytes.  Pure host computation. */
int aw4_workspace_bytes(const aw4_config* cfg, uint64_t* out_bytes);

/* Weights: a new model holds none.  Every call that runs the model (prefill,
 * decode, verify, draft, batch decode, aw4_decode_hidden, aw4_time_phase)
 * returns AW4_E_STATE until every tensor of its config (aw4_tensor_shape; the
 * draft head's and its map included when draft_vocab > 0) has been given values
 * by aw4_quantize_tensor (all rows, over one or more calls), aw4_load_tensor,
 * aw4_set_vector, aw4_set_draft_map or aw4_load_weights. */

/* Bind a model to a caller-owned device arena of at least
 * aw4_workspace_bytes() bytes, 256-byte aligned, on the current HIP device,
 * and to hip_stream (a hipStream_t; NULL = the null stream).  The arena stays
 * owned by the caller and must outlive the model.  The library allocates no
 * device memory.  Zeroes states and caches (enqueued on the stream).
 * Errors: AW4_E_INVAL, AW4_E_ARENA, AW4_E_NODEVICE, AW4_E_HIP. */
int aw4_create(const aw4_config* cfg, void* dev_arena, uint64_t arena_bytes, void* hip_stream,
               aw4_model** out_model);

/* Release host-side resources (captured graphs included).  NULL is a no-op. */
void aw4_destroy(aw4_model* model);

const char* aw4_status_string(int status);
const char* aw4_last_error(const aw4_model* model);

/* ----------------------------------------------------------- weights */

/* Shape of a tensor kind (layer -1 for the global ones). */
int aw4_tensor_shape(const aw4_model* model, int32_t layer, int32_t kind, int64_t* rows, int64_t* cols);

/* Quantise fp32 rows [row0, row0+nrows) of a matrix (kinds 0..5) held at
 * dev_src ([nrows x cols], row-major, device) into the model with the group
 * codec: per 32 consecutive inputs of a row s = fp16(amax / qmax) (qmax 7 for
 * W4, 127 for LM_HEAD, quotient in fp32, round to nearest even), codes
 * clamp(rint(w / s), -qmax, qmax), 0 where s == 0.  Enqueued on the stream. */
int aw4_quantize_tensor(aw4_model* model, int32_t layer, int32_t kind, int64_t row0, int64_t nrows,
                        const float* dev_src);

/* Load an already-quantised matrix from host memory in the logical format:
 * W4: codes uint8 [rows][cols/2], element k in the low nibble of byte k/2 when
 * k is even and the high nibble when odd, nibble = code + 8; LM_HEAD: codes
 * int8 [rows][cols]; scales fp16 bits [rows][cols/32].  Synchronous. */
int aw4_load_tensor(aw4_model* model, int32_t layer, int32_t kind, const void* host_codes,
                    const uint16_t* host_scales);

/* Read a matrix back in the logical format above (test and export use).
 * Synchronous. */
int aw4_export_tensor(aw4_model* model, int32_t layer, int32_t kind, void* host_codes, uint16_t* host_scales);

/* Set a vector kind (6..11, 13..15) from n host floats.  Synchronous. */
int aw4_set_vector(aw4_model* model, int32_t layer, int32_t kind, const float* host_vals, int32_t n);

/* The draft head's vocabulary map (page 5, point 四: the draft head's output
 * projection covers only the most useful ids, 65,536 of about 248K in the
 * pages' model): n == draft_vocab distinct ids in [0, vocab), any order; the
 * library keeps them ascending, which fixes the order of the mapped scores and
 * of the draft draw.  Synchronous.  Errors: AW4_E_INVAL, AW4_E_STATE (no draft
 * head). */
int aw4_set_draft_map(aw4_model* model, const int32_t* host_ids, int32_t n);

/* Weight blob, the host-side form of a whole model (every weight of the
 * stack streams from memory once per decoded token, page 5, bs178.com
 * llamAmpere article, "为什么它真能这么快" point 二, so the weights are loaded
 * once into device memory and stay there).  Layout, little-endian:
 *   "AW4W" magic; uint32 version 4;
 *   int32 x 12: hidden, ffn, vocab, n_layers, gdn_qk_heads, gdn_v_heads,
 *     gdn_head_dim, attn_q_heads, attn_kv_heads, attn_head_dim, group,
 *     draft_vocab (the fields that fix tensor shapes; max_ctx, max_verify,
 *     rms_eps, max_batch and kv_window are run-time choices, not echoed);
 *   char[128] layer_pattern, NUL padded;
 *   uint32 tensor count; then per tensor int32 layer, int32 kind, int64 rows,
 *     int64 cols, uint64 payload bytes, and the payload: a matrix's logical
 *     codes (the aw4_load_tensor format) then its fp16 scale bits [rows][cols/32];
 *     a vector's cols fp32 values; DRAFT_MAP's cols int32 ids.
 * A blob may hold any subset of the config's tensors, each at most once. */

/* Pure host check of a blob against cfg; reads [host_blob, host_blob + bytes)
 * only and enqueues nothing.  AW4_E_FORMAT on a bad magic or version, a config
 * echo that differs from cfg, a tensor the config does not have or with the
 * wrong shape, a duplicated tensor, a payload size that does not match, a
 * truncated blob or bytes after the last tensor, and on values outside the
 * formats: W4 code -8 (nibble 0) or int8 code -128 (the codecs use -qmax..qmax),
 * a negative or non-finite scale, a non-finite vector value, rotation signs other
 * than +-1, map ids repeated or outside [0, vocab).  AW4_E_INVAL: cfg invalid or
 * host_blob NULL with bytes > 0. */
int aw4_check_blob(const aw4_config* cfg, const void* host_blob, uint64_t bytes);

/* Load the tensors of a blob (format above) into the model: the whole blob is
 * checked first (aw4_check_blob against the model's config), so a bad blob
 * returns AW4_E_FORMAT and changes nothing; then every tensor is copied and
 * repacked into the device layout.  Synchronous.  Errors: AW4_E_FORMAT,
 * AW4_E_INVAL, AW4_E_HIP. */
int aw4_load_weights(aw4_model* model, const void* host_blob, uint64_t bytes);

/* ----------------------------------------------------------- decode */

/* Clear recurrent states and caches; position 0.  Enqueued. */
int aw4_reset(aw4_model* model);

/* Append n prompt tokens (positions pos..pos+n-1) through every layer: per
 * token, what a decode step computes (the pages report prompt processing apart
 * from generation: page 3 "Qwen3.8-27B 實測" and page 4, jdon.com, where a
 * 100K-token input takes about two minutes).  host_tokens: n ids in
 * [0, vocab), read during the call.  If dev_logits (device, fp32 [vocab]) is
 * not NULL it receives the logits after the last token.  With a draft head,
 * prefill also gives it one cache entry per prompt position except the last
 * (that position's hidden state and the next prompt token).  Enqueued.
 * Errors: AW4_E_INVAL, AW4_E_CTX_FULL, AW4_E_TOKEN, AW4_E_STATE (vocab 0,
 * weights not complete, or a recent window that must be re-imported). */
int aw4_prefill(aw4_model* model, const int32_t* host_tokens, int32_t n, float* dev_logits);

/* Prompt tokens per prefill chunk.  aw4_prefill runs a prompt in chunks of up
 * to n tokens: each chunk goes through every layer together (the W4 matrices
 * read once per chunk on the matrix cores, the GDN recurrence over the
 * chunk's tokens in order, attention over the cache with causal masks), with
 * the same per-token arithmetic as a decode step.  n = 0 runs the prompt token
 * by token through the decode step.  The default and the maximum is
 * min(1024, max_ctx); shapes whose matrix row lengths are not multiples of 64
 * have no chunked path (maximum 0).  Errors: AW4_E_INVAL. */
int aw4_set_prefill_chunk(aw4_model* model, int32_t n);

/* One decode step on `token` at the current position (the single-user,
 * batch-1 generation step whose speed the pages measure and tie to the bytes
 * streamed per token: page 5, point 二; page 3 "部署前必知" for the 48 GDN +
 * 16 attention layers): embed, all layers (appending this position to the
 * caches), final norm, output head, argmax (lowest index on ties).
 * dev_logits (optional, device) receives fp32 [vocab]; host_argmax (optional)
 * receives the argmax after a stream sync; without it the call only enqueues.
 * Errors: AW4_E_TOKEN, AW4_E_CTX_FULL, AW4_E_STATE (vocab 0, weights not
 * complete, or a recent window that must be re-imported), AW4_E_HIP. */
int aw4_decode_step(aw4_model* model, int32_t token, float* dev_logits, int32_t* host_argmax);

/* n greedy steps starting from first_token (page 5, point 二: decode speed is
 * set by the bytes streamed per token); each step's argmax feeds the next on
 * the device.  host_tokens_out (host, n int32) receives the n generated tokens
 * (one sync at the end).  This is the measured decode loop.  Errors as
 * aw4_decode_step. */
int aw4_decode_greedy(aw4_model* model, int32_t first_token, int32_t n_steps, int32_t* host_tokens_out);

/* Draft verification (page 5, bs178.com llamAmpere article, point 四: the
 * model's draft head proposes k tokens, the target checks them in one pass and
 * keeps each with probability min(1, p/q), which leaves the output distribution
 * equal to the target's).  host_tokens holds k + 1 ids: the last emitted token
 * t0 (not yet run through the model) and k drafts, 0 <= k <= max_verify - 1.
 * The pass runs the k + 1 tokens at positions pos .. pos + k with one sweep
 * over the weights.  With temperature > 0, p_j = softmax(L_j / T) where L_j is
 * the output at position pos + j; draft j+1 is kept when host_u[j] <
 * min(1, p_j(d) / q_j(d)) (dev_q: k rows of V fp32 draft probabilities on the
 * device; a draft with q = 0 is rejected); at the first rejection one token is
 * drawn from max(0, p_j - q_j) renormalised (from p_j if that is all zero), and
 * when every draft is kept a bonus token from p_k, both by inverse CDF in index
 * order with host_u[k].  temperature == 0 is exact-match greedy (dev_q, host_u
 * unused).  host_out receives the accepted drafts followed by the drawn token
 * (*host_n_out = accepted + 1 <= k + 1); the model commits positions pos ..
 * pos + accepted (recurrent states replayed from the committed state, the
 * cache length set), and the last emitted token becomes the next pass's t0.
 * Synchronous.  Errors: AW4_E_INVAL, AW4_E_TOKEN, AW4_E_CTX_FULL, AW4_E_STATE.
 * The committed positions' hidden states stay on the device for the next
 * aw4_draft call. */
int aw4_verify_k(aw4_model* model, const int32_t* host_tokens, int32_t k, const float* dev_q, const float* host_u,
                 float temperature, int32_t* host_out, int32_t* host_n_out);

/* Draft k tokens with the model's draft head (page 5, point 四: depth 3, the
 * draft head scores only the mapped ids).  t0 is the last emitted token, the
 * one the next verify_k (or decode step) runs first.  The call first gives the
 * draft head's cache one entry per position committed since the last draft
 * call by verify_k (that position's hidden state and the token that followed
 * it) plus the entry of the last committed position with t0, in one pass
 * (at most max_verify entries), and draws draft 1 from that last entry; drafts
 * 2..k come from the draft head's own output and the previous draft, in cache
 * entries that are not committed.  A plain decode step feeds nothing: its
 * position is simply absent from the draft cache.
 * Selection: temperature 0 takes the mapped id with the largest score (lowest
 * id on ties); temperature T > 0 draws from q = softmax(score / T) over the
 * mapped ids by inverse CDF in ascending-id order with host_u[j] (k uniforms in
 * [0, 1)), and dev_q (optional, device, [k][vocab] fp32) receives q with zeros
 * outside the map: the draft probabilities verify_k takes.  dev_scores
 * (optional, device, [k][draft_vocab] fp32) receives the mapped scores in
 * ascending-id order.  host_drafts receives the k ids.  1 <= k <= min(3,
 * max_verify - 1).  Synchronous.  Errors: AW4_E_INVAL, AW4_E_TOKEN,
 * AW4_E_CTX_FULL (draft cache), AW4_E_STATE (no draft head, no map, or nothing
 * committed since the last draft call: reset, set_pos and another aw4_draft
 * leave no hidden state to draft from). */
int aw4_draft(aw4_model* model, int32_t t0, int32_t k, float temperature, const float* host_u, float* dev_q,
              float* dev_scores, int32_t* host_drafts);

/* Layers only, at the current position: dev_x_out = stack(dev_x_in), both
 * fp32 [hidden] device vectors (may alias).  For models without a vocabulary
 * (single-layer workloads) and for hidden-state checks.  Enqueued.  Errors:
 * AW4_E_CTX_FULL, AW4_E_STATE (weights not complete). */
int aw4_decode_hidden(aw4_model* model, const float* dev_x_in, float* dev_x_out);

/* Copy the residual vector after the last step's layers (fp32 [hidden]) to the
 * host.  Synchronous. */
int aw4_read_hidden(aw4_model* model, float* host_x);

/* Use (1) or not (0) a captured HIP graph for the per-token launch sequence
 * of decode_step / decode_greedy (default 1). */
int aw4_set_graph(aw4_model* model, int32_t enable);

/* Kernel timing for roofline reports.  Launches one phase of the step `reps`
 * times, cycling through the layers so that consecutive launches stream
 * different weights, between two HIP events on the model's stream (as one
 * captured graph when graphs are enabled, as the decode step runs, except
 * the prefill GEMM phase; the three decode GEMV phases are timed in context:
 * each timed launch follows a launch of the GEMV that precedes it in the
 * step, with events inside the graph around the timed launch alone), and
 * returns the average launch-to-launch duration (microseconds) and the
 * algorithmic work of one launch: the bytes it moves (weights + scales +
 * activations read and written) for the decode phases, the flops (2 M N K) for
 * the prefill GEMM phase.  Synchronous.  Leaves activations scratch
 * overwritten. */
enum {
    AW4_PHASE_FFN_GATE_UP = 0,   /* RMSNorm + gate/up W4 GEMV + SwiGLU  */
    AW4_PHASE_FFN_DOWN = 1,      /* down W4 GEMV + residual add          */
    AW4_PHASE_MIX_IN = 2,        /* RMSNorm + mixer input W4 GEMV         */
    AW4_PHASE_HEAD = 3,          /* final norm + int8 head over the vocab */
    AW4_PHASE_DRAFT_HEAD = 4,    /* draft output norm + int8 head over the mapped ids */
    AW4_PHASE_PREFILL_GATE_UP = 5 /* gate/up W4 GEMM + SwiGLU over a full prefill chunk */
};
int aw4_time_phase(aw4_model* model, int32_t phase, int32_t reps, float* avg_us, uint64_t* bytes_per_launch);

/* Streaming-read bandwidth of the device, the measured reference beside the
 * 8 TB/s peak in bandwidth reports: reps launches of a plain read kernel (512
 * workgroups, each reading one contiguous chunk with eight 4 KB workgroup loads
 * of 16-byte non-temporal words in flight) over bytes (a multiple of 16) at
 * dev_src, timed between two HIP events on hip_stream after one untimed launch;
 * *avg_us receives the average launch duration.  dev_sink: at least 8 KB of
 * device memory the kernel writes.  Synchronous.  Errors: AW4_E_INVAL, AW4_E_HIP. */
int aw4_time_stream_read(const void* dev_src, uint64_t bytes, void* dev_sink, void* hip_stream, int32_t reps,
                         float* avg_us);

/* ----------------------------------------------------------- state */

int aw4_get_pos(aw4_model* model, int32_t* pos);

/* Set the position without touching the caches (state import).  With a
 * recent window, moving the position back leaves ring slots that hold later
 * positions: unless every attention layer's ring was imported since the last
 * decode call, decoding then returns AW4_E_STATE until each ring is imported
 * again (aw4_import_state_win). */
int aw4_set_pos(aw4_model* model, int32_t pos);

/* Sequences (max_batch > 1): the model holds max_batch independent sequences,
 * each with its own recurrent states, caches (the draft head's too) and
 * position.  Every single-sequence call (prefill, decode, verify, draft, the
 * state calls, set_pos) works on the selected one (0 at creation); selecting
 * another keeps each sequence's state.  AW4_E_INVAL outside [0, max_batch). */
int aw4_select_sequence(aw4_model* model, int32_t s);

/* One decode step for each of sequences 0 .. B-1 (1 <= B <= max_batch) with
 * one sweep over the weights (page 3 "Qwen3.8-27B 實測": several users served
 * by one card, four the sweet spot of a 32 GB card): token b runs at sequence
 * b's position through every layer against that sequence's states and cache,
 * then the output head; host_argmax receives the B greedy tokens (lowest
 * index on ties) and each sequence's position advances by one.  The draft
 * head is not fed.  B = 1 with sequence 0 selected runs the single-token
 * step (aw4_decode_step), whose kernels are built for one input vector.
 * Synchronous.  Errors: AW4_E_INVAL, AW4_E_TOKEN, AW4_E_CTX_FULL,
 * AW4_E_STATE (vocab 0). */
int aw4_decode_batch(aw4_model* model, const int32_t* host_tokens, int32_t B, int32_t* host_argmax);

/* Committed entries of the draft head's cache; set it after importing that
 * cache (layer n_layers of the state calls below).  AW4_E_STATE without a draft
 * head. */
int aw4_get_draft_pos(aw4_model* model, int32_t* dpos);
int aw4_set_draft_pos(aw4_model* model, int32_t dpos);

/* GDN recurrent state of one 'G' layer, fp32 [v_heads][head_dim][head_dim]
 * (row i of a head's matrix maps keys to value dim i).  Synchronous. */
int aw4_export_state_gdn(aw4_model* model, int32_t layer, float* host_S);
int aw4_import_state_gdn(aw4_model* model, int32_t layer, const float* host_S);

/* Cache of one 'A' layer (or, as layer n_layers, of the draft head), entries
 * [0, npos), logical layout: K codes int8
 * [npos][kv_heads][head_dim], K scales fp16 [npos][kv_heads][head_dim/32],
 * V codes int8 in -3..3 (rotated domain) [npos][kv_heads][head_dim], V scales
 * fp16 [npos][kv_heads][head_dim/32].  Synchronous. */
int aw4_export_state_kv(aw4_model* model, int32_t layer, int32_t npos, int8_t* host_kc, uint16_t* host_ks,
                        int8_t* host_vc, uint16_t* host_vs);
int aw4_import_state_kv(aw4_model* model, int32_t layer, int32_t npos, const int8_t* host_kc,
                        const uint16_t* host_ks, const int8_t* host_vc, const uint16_t* host_vs);

/* The recent-window ring of attention layer `layer` (kv_window > 0), in the
 * logical layout: keys and rotated values as fp16 bits [kv_window][nkv][dh],
 * position t at slot t % kv_window.  Host buffers of kv_window * nkv * dh
 * uint16 each, owned by the caller.  Synchronises the model's stream.
 * AW4_E_INVAL: not an attention layer, or no window configured. */
int aw4_export_state_win(aw4_model* model, int32_t layer, uint16_t* host_kw, uint16_t* host_vw);
int aw4_import_state_win(aw4_model* model, int32_t layer, const uint16_t* host_kw, const uint16_t* host_vw);

/* ----------------------------------------------------------- no allocation */

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the decode
 * step of aw4_decode_step, with the step's split partials (attention) and the
 * output head's per-block partials in a static device array the library
 * holds (4 MiB per device, kept until the process ends) instead of the arena.
 * The step's kernels are launched one by one (no graph of its own), so a
 * caller may capture them into its own graph; pass host_argmax = NULL under
 * capture (it synchronises the stream).  Every call on a device shares that
 * device's array and its last contents: calls that overlap on one device (two
 * models on one device driven from two threads or streams) race.  A step
 * writes every partial it reads, so nothing needs clearing between calls.
 * Errors: as aw4_decode_step, and AW4_E_INVAL when the step needs more than
 * the 4 MiB (attn_q_heads x split slots x (attn_head_dim + 2) x 4 bytes for
 * the attention partials, plus the head's partials; the 27B shape needs 1.6 MB). */
int aw4_decode_step_static(aw4_model* model, int32_t token, float* dev_logits, int32_t* host_argmax);

/* ----------------------------------------------------------- test hook */

/* Error-path testing: with n >= 1, the n-th checked HIP runtime call the
 * library makes from now on (on any model) is reported as failed, once, and
 * the entry point that made it returns AW4_E_HIP; the call itself has run.
 * n <= 0 disarms.  After an AW4_E_HIP the model's device state is undefined
 * until aw4_reset or a state import.  Not thread-safe across models. */
int aw4_test_fail_hip_call(int32_t n);

#ifdef __cplusplus
}
#endif

#endif /* AW4_H */

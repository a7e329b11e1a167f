"""Synthetic workload definitions: model shapes, seeds and input recipes.

Shapes follow the hybrid stack the reference pages discuss (a dense 27B-class
model with 48 Gated DeltaNet layers and 16 gated-attention layers, vocabulary
about 248K; page 3 "Qwen3.8-27B 實測", section "部署前必知", and page 5, the
bs178.com translation of the llamAmpere post, section "为什么它真能这么快"
point 一).  Sizes the pages leave open are fixed here.

This module holds no arithmetic of the decode step.
"""
from dataclasses import dataclass, field, asdict, replace
import math


@dataclass(frozen=True)
class Shape:
    hidden: int
    ffn: int
    vocab: int
    pattern: str            # one letter per layer: 'G' Gated DeltaNet, 'A' gated attention
    gdn_qk_heads: int
    gdn_v_heads: int
    gdn_head_dim: int
    attn_q_heads: int
    attn_kv_heads: int
    attn_head_dim: int
    group: int = 32
    rms_eps: float = 1e-6
    max_ctx: int = 4096
    max_verify: int = 4
    draft_vocab: int = 0    # ids in the draft head's vocabulary map; 0: no draft head
    max_batch: int = 1      # sequences with their own state (batch decode)
    kv_window: int = 0      # recent positions the attention caches also keep at fp16; 0: none
    kv_format: int = 0      # cache codecs: 0 K int8 + V rotated 3-bit; 1 q4_0 (K, V 4-bit, V not
                            # rotated); 2 K int8 + V rotated 3-bit Lloyd-Max codebook

    @property
    def n_layers(self):
        return len(self.pattern)

    def as_dict(self):
        d = asdict(self)
        d["n_layers"] = self.n_layers
        return d


TOY = Shape(hidden=512, ffn=1536, vocab=4096, pattern="GA", gdn_qk_heads=4, gdn_v_heads=4,
            gdn_head_dim=64, attn_q_heads=4, attn_kv_heads=1, attn_head_dim=64, max_ctx=1024)

# the 27B-shape stack with its built-in draft head, whose output projection
# covers 65,536 of the 248,320 ids (page 5, bs178.com llamAmpere article, point 四)
FULL_27B = Shape(hidden=5120, ffn=17408, vocab=248320, pattern="GGGA" * 16, gdn_qk_heads=16,
                 gdn_v_heads=32, gdn_head_dim=128, attn_q_heads=24, attn_kv_heads=4,
                 attn_head_dim=256, max_ctx=16384, draft_vocab=65536)

# the toy stack with a draft head over a quarter of its vocabulary
TOY_MTP = replace(TOY, draft_vocab=1024)

# Single full-size layers (vocab 0: no embedding and no lm_head, the layer runs on
# hidden vectors).  pattern length = number of independent weight copies.
GDN_LAYER = replace(FULL_27B, vocab=0, pattern="G", max_ctx=16, draft_vocab=0)
ATTN_LAYER = replace(FULL_27B, vocab=0, pattern="A", max_ctx=4096 + 512, draft_vocab=0)


def with_(shape, **kw):
    return replace(shape, **kw)


# ---------------------------------------------------------------- weight recipe
# tensor kinds (numbering shared by the C ABI, the oracle and this recipe)
T_MIX_IN, T_MIX_OUT, T_FFN_GATE, T_FFN_UP, T_FFN_DOWN, T_LM_HEAD = 0, 1, 2, 3, 4, 5
T_NORM_MIX, T_NORM_FFN, T_NORM_GATED, T_A_BIAS, T_NORM_FINAL, T_RHT_SIGNS = 6, 7, 8, 9, 10, 11
# draft head, all at layer index n_layers (beside its gated-attention layer's kinds 0-4, 6, 7)
T_DRAFT_FUSE, T_DRAFT_NORM_EMB, T_DRAFT_NORM_HID, T_DRAFT_NORM_OUT, T_DRAFT_MAP = 12, 13, 14, 15, 16

W4, I8, VEC, SIGNS, MAP = "w4", "i8", "vec", "signs", "map"

WEIGHT_STD = 0.02       # "weights N(0, 0.02)", read as a standard deviation
A_BIAS = 2.0            # alpha = sigmoid(a + 2): a ~ N(2, 0.5) once x is unit-RMS


def stream_id(layer, kind):
    """Philox stream of one tensor: layer -1 holds the global tensors."""
    return ((layer + 1) << 8) | kind


@dataclass
class TensorSpec:
    layer: int
    kind: int
    fmt: str
    rows: int
    cols: int
    # (row_start, row_end, sigma) segments for normal-filled matrices
    segments: list = field(default_factory=list)
    const: float = None      # constant vectors
    jitter: float = 0.0      # vectors: 1 + jitter * z

    @property
    def stream(self):
        return stream_id(self.layer, self.kind)


def mixer_in_rows(s: Shape, kind_char):
    if kind_char == "G":
        qk = s.gdn_qk_heads * s.gdn_head_dim
        v = s.gdn_v_heads * s.gdn_head_dim
        return 2 * qk + 2 * v + 2 * s.gdn_v_heads
    qd = s.attn_q_heads * s.attn_head_dim
    kvd = s.attn_kv_heads * s.attn_head_dim
    return 2 * qd + 2 * kvd


def mixer_out_cols(s: Shape, kind_char):
    if kind_char == "G":
        return s.gdn_v_heads * s.gdn_head_dim
    return s.attn_q_heads * s.attn_head_dim


def tensor_specs(s: Shape, norm_jitter=0.0):
    """Every tensor of the model, in load order."""
    H = s.hidden
    out = []
    for li, t in enumerate(s.pattern):
        rows = mixer_in_rows(s, t)
        if t == "G":
            nv = s.gdn_v_heads
            main = rows - 2 * nv
            segs = [(0, main, WEIGHT_STD), (main, main + nv, 0.5 / math.sqrt(H)),
                    (main + nv, main + 2 * nv, 1.0 / math.sqrt(H))]
        else:
            segs = [(0, rows, WEIGHT_STD)]
        out.append(TensorSpec(li, T_MIX_IN, W4, rows, H, segs))
        oc = mixer_out_cols(s, t)
        out.append(TensorSpec(li, T_MIX_OUT, W4, H, oc, [(0, H, WEIGHT_STD)]))
        out.append(TensorSpec(li, T_FFN_GATE, W4, s.ffn, H, [(0, s.ffn, WEIGHT_STD)]))
        out.append(TensorSpec(li, T_FFN_UP, W4, s.ffn, H, [(0, s.ffn, WEIGHT_STD)]))
        out.append(TensorSpec(li, T_FFN_DOWN, W4, H, s.ffn, [(0, H, WEIGHT_STD)]))
        out.append(TensorSpec(li, T_NORM_MIX, VEC, 1, H, jitter=norm_jitter))
        out.append(TensorSpec(li, T_NORM_FFN, VEC, 1, H, jitter=norm_jitter))
        if t == "G":
            out.append(TensorSpec(li, T_NORM_GATED, VEC, 1, s.gdn_head_dim, jitter=norm_jitter))
            out.append(TensorSpec(li, T_A_BIAS, VEC, 1, s.gdn_v_heads, const=A_BIAS))
    if s.vocab > 0:
        out.append(TensorSpec(-1, T_LM_HEAD, I8, s.vocab, H, [(0, s.vocab, WEIGHT_STD)]))
        out.append(TensorSpec(-1, T_NORM_FINAL, VEC, 1, H, jitter=norm_jitter))
    if "A" in s.pattern or s.draft_vocab > 0:
        out.append(TensorSpec(-1, T_RHT_SIGNS, SIGNS, 1, s.attn_head_dim))
    if s.draft_vocab > 0:
        D = s.n_layers
        rows = mixer_in_rows(s, "A")
        out.append(TensorSpec(D, T_MIX_IN, W4, rows, H, [(0, rows, WEIGHT_STD)]))
        out.append(TensorSpec(D, T_MIX_OUT, W4, H, mixer_out_cols(s, "A"), [(0, H, WEIGHT_STD)]))
        out.append(TensorSpec(D, T_FFN_GATE, W4, s.ffn, H, [(0, s.ffn, WEIGHT_STD)]))
        out.append(TensorSpec(D, T_FFN_UP, W4, s.ffn, H, [(0, s.ffn, WEIGHT_STD)]))
        out.append(TensorSpec(D, T_FFN_DOWN, W4, H, s.ffn, [(0, H, WEIGHT_STD)]))
        out.append(TensorSpec(D, T_NORM_MIX, VEC, 1, H, jitter=norm_jitter))
        out.append(TensorSpec(D, T_NORM_FFN, VEC, 1, H, jitter=norm_jitter))
        out.append(TensorSpec(D, T_DRAFT_FUSE, W4, H, 2 * H, [(0, H, WEIGHT_STD)]))
        out.append(TensorSpec(D, T_DRAFT_NORM_EMB, VEC, 1, H, jitter=norm_jitter))
        out.append(TensorSpec(D, T_DRAFT_NORM_HID, VEC, 1, H, jitter=norm_jitter))
        out.append(TensorSpec(D, T_DRAFT_NORM_OUT, VEC, 1, H, jitter=norm_jitter))
        out.append(TensorSpec(D, T_DRAFT_MAP, MAP, 1, s.draft_vocab))
    return out


# ---------------------------------------------------------------- other streams
STREAM_PROMPT = 0x00F00001
STREAM_HIDDEN = 0x00F00002      # per-step hidden inputs of the single-layer workloads
STREAM_UNIFORM = 0x00F00003
STREAM_DRAFT = 0x00F00004
STREAM_MAP = 0x00F00005         # the draft head's vocabulary map
STREAM_STATE = 0x00F00100       # + small offsets for the synthetic cache fill
DRAFT_LOGIT_STD = 1.43          # about 0.02 * sqrt(5120), the spread of random-weight logits

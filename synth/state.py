"""Synthetic decode state (recurrent states and compressed KV cache), seeded.

Used where a long context has to exist without prefilling it token by token
(8K-262K positions): both the oracle and the GPU model import the same arrays.
Codes and scales are drawn directly (discretised normals, fp16 bit patterns),
so no quantiser is involved (the recent-window ring, when the shape has one,
is fp16 of seeded normals).  Magnitudes mimic what the decode step writes:
keys ~ N(0, 1.4^2) stored as int8 codes x 0.035, rotated values ~ 1.4 in
3-bit codes x ~1, recurrent state entries ~ N(0, 0.1^2).
"""
import numpy as np

from . import codes, normal, scale_bits
from .workloads import STREAM_STATE

K_SPREAD256 = 40 * 256          # code std ~ 40 (keys of std 1.4 at scale 0.035)
V_SPREAD256 = 358               # code std ~ 1.4
K_SCALE_BITS = 0x287B           # fp16 0.0350
V_SCALE_BITS = 0x3C00           # fp16 1.0
S_STD = 0.1


def _stream(layer, part):
    return STREAM_STATE + layer * 8 + part


def gdn_state(shape, layer, seed):
    n = shape.gdn_v_heads * shape.gdn_head_dim
    return normal(n, shape.gdn_head_dim, S_STD, seed, _stream(layer, 0)).reshape(
        shape.gdn_v_heads, shape.gdn_head_dim, shape.gdn_head_dim)


# the 4-bit cache (format 1): code std ~ 2.8 (keys and values of std 1.4 at scale 0.5)
Q4_SPREAD256 = 720
Q4_SCALE_BITS = 0x3800          # fp16 0.5


def kv_state(shape, layer, npos, seed):
    """Logical cache codes and scales of npos positions in the shape's cache
    format: format 0 int8 keys and 3-bit values (-3..3); format 1 4-bit keys
    and values (-7..7); format 2 int8 keys and codebook indices 0..7 (from
    discretised normals folded onto the eight levels)."""
    d, nkv = shape.attn_head_dim, shape.attn_kv_heads
    fmt = getattr(shape, "kv_format", 0)
    n = npos * nkv * d
    if fmt == 1:
        kc = codes(n, Q4_SPREAD256, 7, seed, _stream(layer, 1)).reshape(npos, nkv, d)
        vc = codes(n, Q4_SPREAD256, 7, seed, _stream(layer, 2)).reshape(npos, nkv, d)
        kb, vb = Q4_SCALE_BITS, Q4_SCALE_BITS
    else:
        kc = codes(n, K_SPREAD256, 127, seed, _stream(layer, 1)).reshape(npos, nkv, d)
        kb, vb = K_SCALE_BITS, V_SCALE_BITS
        if fmt == 2:
            a = codes(n, V_SPREAD256, 7, seed, _stream(layer, 2))
            vc = np.where(a >= 0, np.minimum(a, 3) + 4, np.maximum(a, -4) + 4).astype(np.int8).reshape(npos, nkv, d)
        else:
            vc = codes(n, V_SPREAD256, 3, seed, _stream(layer, 2)).reshape(npos, nkv, d)
    ks = scale_bits(n // 32, kb, seed, _stream(layer, 3)).reshape(npos, nkv, d // 32)
    vs = scale_bits(n // 32, vb, seed, _stream(layer, 4)).reshape(npos, nkv, d // 32)
    return kc, ks, vc, vs


def win_state(shape, layer, seed):
    """Recent-window ring [W][nkv][d] as fp16 bits: keys ~ N(0, 1.4^2), rotated
    values ~ N(0, 1), the magnitudes the codes above stand for."""
    d, nkv, W = shape.attn_head_dim, shape.attn_kv_heads, shape.kv_window
    kw = normal(W * nkv, d, 1.4, seed, _stream(layer, 5)).astype(np.float16).view(np.uint16)
    vw = normal(W * nkv, d, 1.0, seed, _stream(layer, 6)).astype(np.float16).view(np.uint16)
    return kw.reshape(W, nkv, d), vw.reshape(W, nkv, d)


def fill(model, shape, npos, seed, gdn=True, kv=True, draft=True):
    """Import a synthetic state of npos positions into a model exposing
    import_gdn / import_kv / set_pos (the GPU binding) or set_gdn_state /
    set_kv / set_pos (the oracle).  With a draft head, its cache gets npos - 1
    entries (one per position whose next token is known) of the same recipe."""
    put_kv = model.import_kv if hasattr(model, "import_kv") else model.set_kv
    for l, t in enumerate(shape.pattern):
        if t == "G" and gdn:
            S = gdn_state(shape, l, seed)
            (model.import_gdn if hasattr(model, "import_gdn") else model.set_gdn_state)(l, S)
        elif t == "A" and kv:
            put_kv(l, *kv_state(shape, l, npos, seed))
            if getattr(shape, "kv_window", 0) > 0:
                (model.import_win if hasattr(model, "import_win") else model.set_win)(l, *win_state(shape, l, seed))
    if getattr(shape, "draft_vocab", 0) > 0 and draft and npos > 0:
        put_kv(shape.n_layers, *kv_state(shape, shape.n_layers, npos - 1, seed))
        model.set_dpos(npos - 1)
    model.set_pos(npos)

"""Shared test helpers: tiny shapes and model builders from the seeded recipe."""
import numpy as np

import oracle
import synth
from synth import workloads as W

# a tiny hybrid with grouped heads on both mixer types, for brute-force pins
TINY = W.Shape(hidden=128, ffn=192, vocab=160, pattern="GAGA", gdn_qk_heads=2, gdn_v_heads=4,
               gdn_head_dim=64, attn_q_heads=4, attn_kv_heads=2, attn_head_dim=64, max_ctx=64)
# the same with a draft head over 40 of the 160 ids
TINY_MTP = W.with_(TINY, draft_vocab=40)


def logical_weights(shape, seed, norm_jitter=0.0):
    """Logical (codes, scales) of every tensor, quantised by the oracle codec,
    keyed (layer, kind); vectors as float64; signs as int8."""
    out = {}
    for spec in W.tensor_specs(shape, norm_jitter):
        if spec.fmt == W.W4:
            out[(spec.layer, spec.kind)] = oracle.quant_w4(synth.matrix_rows(spec, seed, 0, spec.rows))
        elif spec.fmt == W.I8:
            out[(spec.layer, spec.kind)] = oracle.quant_i8(synth.matrix_rows(spec, seed, 0, spec.rows))
        elif spec.fmt == W.VEC:
            out[(spec.layer, spec.kind)] = synth.vector(spec, seed).astype(np.float64)
        elif spec.fmt == W.MAP:
            out[(spec.layer, spec.kind)] = synth.draft_map(shape, seed)
        else:
            out[(spec.layer, spec.kind)] = synth.signs(spec.cols, seed, spec.stream)
    return out


def oracle_from_logical(shape, lw):
    m = oracle.Model(shape)
    for (layer, kind), v in lw.items():
        if kind in (0, 1, 2, 3, 4, W.T_DRAFT_FUSE):
            m.load_w4(layer, kind, *v)
        elif kind == 5:
            m.load_i8(*v)
        elif kind == 11:
            m.load_signs(v)
        elif kind == W.T_DRAFT_MAP:
            m.set_draft_map(v)
        else:
            m.load_vec(layer, kind, v)
    return m


def rel_l2(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))

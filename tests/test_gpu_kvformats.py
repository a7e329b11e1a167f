"""GPU parity of the KV-cache variants (kv_format 1: q4_0, keys and values
4-bit per 32, values not rotated; kv_format 2: int8 keys, rotated values coded
with the 8-level Lloyd-Max Gaussian codebook) against the oracle with the same
format: teacher-forced toy steps (outputs and the appended codes, every code
difference at the oracle's own rounding or nearest-level tie), free-running
greedy decoding, and the full-size attention layer (d = 256, 6 q heads per kv
head) on synthetic 4096- and 131,071-position caches; the variants' refusals."""
import sys

import numpy as np
import pytest

import oracle
import synth
from synth import state as SS
from synth import workloads as W
from tests.helpers import rel_l2
from tests.test_gpu_parity import TOL, TOL_STEP, _tie_checked, _layer_pair

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def aw4():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import attention_w4_amd as A
    A.lib()
    return A


def _gpu_model(A, shape, seed):
    from synth.gpu_load import load_recipe
    m = A.Model(shape)
    load_recipe(m, shape, seed)
    return m


def _import(gm, om, shape):
    for l, t in enumerate(shape.pattern):
        if t == "G":
            gm.import_gdn(l, om.get_gdn_state(l).astype(np.float32))
        else:
            gm.import_kv(l, *om.get_kv(l, om.pos))
    gm.set_pos(om.pos)


def _f16(b):
    return float(np.asarray(b, np.uint16).view(np.float16))


def _lm_tie_checked(gc, oc, gs, os_, vals, rel_tol=1e-3):
    """codebook codes [n][32] / scales [n] of one append with the oracle's fp32
    (rotated) values: a differing scale must sit at an fp16 rounding tie of the
    group's root mean square, a differing code must be the neighbouring index
    with v / s at the midpoint of the two levels; returns the differences"""
    lv = oracle.lm_levels()
    bad, nd = [], 0
    for g in range(gc.shape[0]):
        v = vals[g].astype(np.float64)
        rms = float(np.sqrt(np.mean(v * v)))
        if gs[g] != os_[g]:
            mid = 0.5 * (_f16(gs[g]) + _f16(os_[g]))
            if abs(rms - mid) > rel_tol * rms:
                bad.append(("scale", g, rms, _f16(gs[g]), _f16(os_[g])))
            nd += int(np.sum(gc[g] != oc[g]))
            continue
        s = _f16(os_[g])
        for i in np.nonzero(gc[g] != oc[g])[0]:
            nd += 1
            a, b = int(gc[g][i]), int(oc[g][i])
            t = float(v[i]) / s
            mid = 0.5 * (lv[min(a, b)] + lv[max(a, b)])
            if abs(a - b) != 1 or abs(t - mid) > rel_tol * 2.2 + 1e-3:
                bad.append(("code", g, i, t, a, b))
    assert not bad, bad[:5]
    return nd


@pytest.mark.parametrize("fmt", [1, 2])
def test_kvformat_toy_teacher_forced(aw4, fmt):
    import torch
    shape = W.with_(W.TOY, kv_format=fmt)
    _say("case: toy stack, cache format", fmt, "teacher-forced 40 steps")
    om = oracle.from_recipe(shape, 3)
    gm = _gpu_model(aw4, shape, 3)
    toks = synth.tokens(40, shape.vocab, 3)
    logits = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    clean, tied = [], []
    for i in range(40):
        t = int(toks[i])
        _import(gm, om, shape)
        pos = om.pos
        xo, lo, ao = om.decode_token(t)
        ag = gm.decode_step(t, logits)
        xg, lg = gm.read_hidden(), logits.cpu().numpy()
        err = max(rel_l2(xg, xo), rel_l2(lg, lo))
        flips = 0
        for l, lt in enumerate(shape.pattern):
            if lt != "A" or flips:
                continue
            gk, ok = gm.export_kv(l, pos + 1), om.get_kv(l, pos + 1)
            kv, vv = om.last_kv(l)
            flips += _tie_checked(gk[0][pos].reshape(-1, 32), ok[0][pos].reshape(-1, 32), gk[1][pos].ravel(),
                                  ok[1][pos].ravel(), kv.reshape(-1, 32), 7 if fmt == 1 else 127)
            if fmt == 1:
                flips += _tie_checked(gk[2][pos].reshape(-1, 32), ok[2][pos].reshape(-1, 32), gk[3][pos].ravel(),
                                      ok[3][pos].ravel(), vv.reshape(-1, 32), 7)
            else:
                flips += _lm_tie_checked(gk[2][pos].reshape(-1, 32), ok[2][pos].reshape(-1, 32), gk[3][pos].ravel(),
                                         ok[3][pos].ravel(), vv.reshape(-1, 32))
        if ag != ao:
            top = np.sort(lo)[-2:]
            assert top[1] - top[0] < 1e-3 * np.std(lo), (i, ag, ao)
        (tied if flips else clean).append(err)
    _say(f"clean steps {len(clean)} worst {max(clean):.2e}; steps with tie flips {len(tied)}")
    assert len(clean) >= 20
    assert max(clean) < TOL_STEP
    assert not tied or max(tied) < 0.1
    gm.close()


@pytest.mark.parametrize("fmt", [1, 2])
def test_kvformat_toy_free_running(aw4, fmt):
    shape = W.with_(W.TOY, kv_format=fmt)
    _say("case: toy stack, cache format", fmt, "64-token prompt + 64 greedy steps")
    prompt = synth.tokens(64, shape.vocab, 8)
    gm = _gpu_model(aw4, shape, 8)
    gm.prefill(prompt[:-1])
    got = list(gm.decode_greedy(int(prompt[-1]), 64))
    xg = gm.read_hidden()
    gm.close()
    om = oracle.from_recipe(shape, 8)
    for t in prompt[:-1]:
        om.decode_token(int(t))
    tok, ref = int(prompt[-1]), []
    for _ in range(64):
        x, _, tok = om.decode_token(tok)
        ref.append(tok)
    _say(f"tokens equal {got == ref}, hidden rel-L2 {rel_l2(xg, x):.2e}")
    assert got == ref
    assert rel_l2(xg, x) < TOL


@pytest.mark.parametrize("fmt,npos", [(1, 4096), (2, 4096), (1, 131071), (2, 131071)])
def test_kvformat_attention_layer_full_size(aw4, fmt, npos):
    """full-size gated-attention layer on a synthetic cache in the format,
    teacher-forced"""
    _say("case: full-size attention layer, cache format", fmt, "positions", npos)
    shape = W.with_(W.ATTN_LAYER, max_ctx=npos + 64, kv_format=fmt)
    w = _layer_pair(aw4, shape, 5, 4 if npos < 8192 else 2, npos=npos)
    _say(f"worst layer-delta rel-L2 {w:.2e}")
    assert w < TOL


def test_kvformat_refusals(aw4):
    shape = W.with_(W.TOY, kv_format=1)
    gm = _gpu_model(aw4, shape, 2)
    with pytest.raises(aw4.AW4Error) as ei:
        gm.verify_k([1, 2], temperature=0.0)
    assert ei.value.code == -1
    gm.close()

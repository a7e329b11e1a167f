"""CPU pins of the oracle's recent-window KV variant: the last W cached
positions are read at fp16 (the fp32 key and the fp32 rotated value rounded
once) instead of from their int8 / 3-bit codes, while every position keeps its
codes (page 3, Qwen3.8-27B 實測, section "RTX 4090 24GB": a 130K setup keeps the
last 2,048 tokens at F16 against attention drift).

Pinned against the numpy brute force (which keeps every position's fp16 pair
and picks by position, not through a ring), closed forms of softmax attention
written here, and the ring's slot rule."""
import numpy as np
import pytest
from scipy.linalg import hadamard
from scipy.special import softmax

import oracle
import synth
from oracle import brute
from synth import workloads as W
from tests.helpers import TINY, logical_weights, oracle_from_logical, rel_l2


def _h(x):
    """fp32 value rounded to fp16, as float64"""
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float16).astype(np.float64)


def _bits(x):
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float16).view(np.uint16)


def _rand_cache(rng, T, d):
    kc = rng.integers(-127, 128, (T, d)).astype(np.int8)
    vc = rng.integers(-3, 4, (T, d)).astype(np.int8)
    ks = np.full((T, d // 32), 0x2000, np.uint16)      # 2^-7
    vs = np.full((T, d // 32), 0x3400, np.uint16)      # 0.25
    return kc, ks, vc, vs


@pytest.mark.parametrize("win", [1, 3, 7])
def test_window_model_matches_brute_force(win):
    shape = W.with_(TINY, kv_window=win)
    lw = logical_weights(shape, seed=21, norm_jitter=0.1)
    om = oracle_from_logical(shape, lw)
    bm = brute.BruteModel(shape, lw)
    toks = synth.tokens(5, shape.vocab, seed=21)
    tok = int(toks[0])
    for step in range(14):
        t = int(toks[step]) if step < len(toks) else tok
        xo, lo, ao = om.decode_token(t)
        xb, lb, ab = bm.decode_token(t)
        assert rel_l2(xo, xb) < 1e-10, step
        assert rel_l2(lo, lb) < 1e-10, step
        assert ao == ab
        tok = ao
    n = om.pos
    for l, t in enumerate(shape.pattern):
        if t != "A":
            continue
        # every position keeps its codes
        kc, ks, vc, vs = om.get_kv(l, n)
        assert np.array_equal(kc, np.stack([e[0] for e in bm.kv[l]]))
        assert np.array_equal(vc, np.stack([e[2] for e in bm.kv[l]]))
        # the ring holds the last W positions at slot t % W
        kw, vw = om.get_win(l)
        for p in range(max(0, n - win), n):
            assert np.array_equal(kw[p % win].view(np.float16).astype(np.float64), bm.kv[l][p][4]), (l, p)
            assert np.array_equal(vw[p % win].view(np.float16).astype(np.float64), bm.kv[l][p][5]), (l, p)


def test_window_changes_the_result():
    """A window of 0 and one of 3 give different hidden states (the window is
    read), and a window at least as long as the sequence equals one longer."""
    lw = logical_weights(TINY, seed=22)
    toks = [int(t) for t in synth.tokens(9, TINY.vocab, seed=22)]
    out = {}
    for win in (0, 3, 9, 12):
        shape = W.with_(TINY, kv_window=win)
        om = oracle_from_logical(shape, lw)
        for t in toks:
            x, _, _ = om.decode_token(t)
        out[win] = x
    assert rel_l2(out[3], out[0]) > 1e-6
    assert rel_l2(out[9], out[12]) == 0.0
    assert rel_l2(out[9], out[3]) > 1e-9


def test_single_position_in_window_returns_its_value():
    """One cached position read from the window: softmax weight 1, so the head
    output is the inverse rotation of the stored fp16 rotated value."""
    rng = np.random.default_rng(31)
    d = 64
    s = synth.signs(d, 5, 11)
    kc, ks, vc, vs = _rand_cache(rng, 1, d)
    vr = rng.standard_normal(d)
    kw = _bits(rng.standard_normal(d))[None]
    vw = _bits(vr)[None]
    out = oracle.attend_head(rng.standard_normal(d), kc, ks, vc, vs, s, kw, vw)
    ref = s * (hadamard(d) @ _h(vr)) / np.sqrt(d)
    assert np.allclose(out, ref, atol=1e-12)


@pytest.mark.parametrize("T,win", [(9, 9), (9, 4), (17, 5), (6, 1)])
def test_window_softmax_closed_form(T, win):
    """Positions T - win .. T - 1 come from the ring (slot t % win), the rest
    from their codes; softmax over all T scores, then the inverse rotation."""
    rng = np.random.default_rng(32 + T + win)
    d = 64
    s = synth.signs(d, 6, 11)
    kc, ks, vc, vs = _rand_cache(rng, T, d)
    kf = rng.standard_normal((T, d)) * 1.3
    vf = rng.standard_normal((T, d))
    kw = np.zeros((win, d), np.uint16)
    vw = np.zeros((win, d), np.uint16)
    for t in range(T):                      # a ring written in position order
        kw[t % win] = _bits(kf[t])
        vw[t % win] = _bits(vf[t])
    q = rng.standard_normal(d)
    out = oracle.attend_head(q, kc, ks, vc, vs, s, kw, vw)
    K = np.where(np.arange(T)[:, None] >= T - win, _h(kf), kc * 2.0 ** -7)
    V = np.where(np.arange(T)[:, None] >= T - win, _h(vf), vc * 0.25)
    p = softmax(K @ q / np.sqrt(d))
    ref = s * (hadamard(d) @ (p @ V)) / np.sqrt(d)
    assert np.allclose(out, ref, atol=1e-12)


def test_window_is_closer_to_unquantised_attention():
    """Reading the recent positions at fp16 brings a head's output closer to
    attention over the unquantised keys and values (the variant's purpose)."""
    rng = np.random.default_rng(33)
    d, T = 256, 48
    s = synth.signs(d, 7, 11)
    k = rng.standard_normal((T, d)) * 1.4
    v = rng.standard_normal((T, d))
    q = rng.standard_normal(d) * 2.0
    codes = [oracle.kv_encode(k[t], v[t], s) for t in range(T)]
    kc, ks, vc, vs = (np.stack([c[i] for c in codes]) for i in range(4))
    vr = np.stack([oracle.rht_forward(v[t], s) for t in range(T)])
    exact = softmax(k @ q / np.sqrt(d)) @ v
    err = {}
    for win in (0, 16, T):
        if win == 0:
            out = oracle.attend_head(q, kc, ks, vc, vs, s)
        else:
            kw = np.stack([_bits(k[t]) for t in range(T)])[T - win:]
            vw = np.stack([_bits(vr[t]) for t in range(T)])[T - win:]
            # ring slots: position t at t % win
            order = np.argsort([t % win for t in range(T - win, T)])
            out = oracle.attend_head(q, kc, ks, vc, vs, s, kw[order], vw[order])
        err[win] = rel_l2(out, exact)
    assert err[T] < err[16] < err[0]
    assert err[T] < 2e-3

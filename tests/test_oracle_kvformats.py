"""Pins of the oracle's KV-cache variants (no GPU needed).

Format 1 (q4_0: keys and values both 4-bit per 32 with an fp16 scale, values
not rotated; page 3 "Qwen3.8-27B 實測", section "RTX 5090 32GB：可以四人", and
page 4, jdon.com, section on 262K contexts) and format 2 (keys int8, values
rotated then coded with the 8-level Lloyd-Max codebook of a unit Gaussian).
Each expected value comes from the mathematics: Lloyd's conditions computed
with scipy's normal distribution, closed forms of attention over one cached
position, the nearest-level rule checked by brute force, and the independent
numpy model in oracle/brute.py.
"""
import numpy as np
import pytest
from scipy.stats import norm

import oracle
import synth
from oracle import brute
from synth import workloads as W
from tests.helpers import TINY, logical_weights, oracle_from_logical, rel_l2


# ------------------------------------------------------------- the codebook
def _lloyd_max(n=8, iters=2000):
    """Lloyd's algorithm for N(0, 1) from uniform starting levels: alternately
    thresholds at midpoints and levels at the conditional means of their cells"""
    lv = np.linspace(-2.0, 2.0, n)
    for _ in range(iters):
        b = np.concatenate([[-np.inf], 0.5 * (lv[1:] + lv[:-1]), [np.inf]])
        mass = norm.cdf(b[1:]) - norm.cdf(b[:-1])
        lv = (norm.pdf(b[:-1]) - norm.pdf(b[1:])) / mass
    return lv


def test_codebook_is_the_gaussian_lloyd_max_quantizer():
    """the codebook's levels satisfy Lloyd's conditions for a unit Gaussian: they
    equal the fixed point of Lloyd's algorithm (computed here from scratch) to
    within fp16 rounding, and its distortion is Max's 0.03454 for eight levels"""
    ref = _lloyd_max()
    lv = oracle.lm_levels()
    assert np.all(np.diff(lv) > 0) and np.array_equal(lv, -lv[::-1])
    assert np.max(np.abs(lv - ref)) < 2e-3, (lv, ref)
    # fp16 values of the levels
    assert np.array_equal(lv, lv.astype(np.float16).astype(np.float64))
    b = np.concatenate([[-np.inf], 0.5 * (ref[1:] + ref[:-1]), [np.inf]])
    dist = sum(
        (norm.expect(lambda x, c=c: (x - c) ** 2, lb=b[i], ub=b[i + 1])) for i, c in enumerate(ref))
    assert abs(dist - 0.03454) < 2e-4
    # the brute model's own copy of the levels is the same codebook
    assert np.array_equal(brute.lm_levels(), lv)


def test_codebook_codec_hand_worked():
    """a group whose mean square is 1 (eight probes plus 24 fillers of equal
    magnitude chosen to make it so): the scale is exactly 1, each probe placed
    on a level returns that level's index, a probe on the midpoint of two
    levels returns the lower one, and the fillers (+-0.8627) land on +-0.7560"""
    lv = oracle.lm_levels()

    def group(probes):
        probes = np.asarray(probes, np.float64)
        f = np.sqrt((32 - np.sum(probes ** 2)) / 24)
        x = np.concatenate([probes, np.tile([f, -f], 12)]).astype(np.float32)
        return x, float(np.float32(f))

    x, f = group(lv)
    sb, c = oracle.quant_group_lm(x)
    assert sb == 0x3C00                           # scale 1.0
    assert list(c[:8]) == list(range(8))
    assert list(c[8:10]) == [5, 2] and abs(f - 0.8627) < 1e-3
    mids = [(lv[3] + lv[4]) / 2, (lv[4] + lv[5]) / 2, (lv[6] + lv[7]) / 2, (lv[0] + lv[1]) / 2]
    x, _ = group(mids + [0.0] * 4)
    sb, c = oracle.quant_group_lm(x)
    assert sb == 0x3C00
    assert list(c[:4]) == [3, 4, 6, 0]
    # an all-zero group: scale 0, every code 4
    s0, c0 = oracle.quant_group_lm(np.zeros(32, np.float32))
    assert s0 == 0 and np.all(c0 == 4)


def test_codebook_codec_is_nearest_level():
    """random groups: every code is the level nearest to x / s (brute force over
    the eight levels in fp64), the scale is fp16 of the root mean square, and
    the numpy model agrees bit for bit"""
    rng = np.random.default_rng(3)
    lv = oracle.lm_levels()
    for _ in range(300):
        x = (rng.standard_normal(32) * 10.0 ** rng.uniform(-3, 2)).astype(np.float32)
        sb, c = oracle.quant_group_lm(x)
        s = float(np.asarray(sb, np.uint16).view(np.float16))
        assert sb == np.float16(np.sqrt(np.float32(np.mean(x.astype(np.float64) ** 2)))).view(np.uint16)
        t = (x / np.float32(s)).astype(np.float64)
        d = np.abs(t[:, None] - lv[None, :])
        best = d.min(axis=1)
        assert np.all(d[np.arange(32), c.astype(int)] == best)
        bc, bs = brute.quant_lm(x[None, :])
        assert np.array_equal(bc[0], c) and bs[0] == sb


def test_codebook_beats_uniform_3bit_on_gaussian_values():
    """what the variant is for: on Gaussian (rotated) values the codebook's
    squared error is below the uniform 3-bit codec's"""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((4000, 32)).astype(np.float32)
    cu, su = brute.quant(x, 3)
    cl, sl = brute.quant_lm(x)
    eu = np.mean((brute.dequant_i8(cu, su) - x) ** 2)
    el = np.mean((brute.dequant_lm(cl, sl) - x) ** 2)
    assert el < 0.85 * eu, (el, eu)
    assert abs(el - 0.0345) < 0.01      # close to Max's distortion (scale estimated per group)


# ------------------------------------------------------------- attention closed forms
@pytest.mark.parametrize("fmt", [1, 2])
def test_one_cached_position_returns_its_value(fmt):
    """with one cached position the head's output is that position's value:
    format 1 the dequantised 4-bit value itself, format 2 the inverse rotation
    of the codebook value"""
    rng = np.random.default_rng(5 + fmt)
    d = 64
    sg = synth.signs(d, seed=2, stream=11)
    k, v, q = rng.standard_normal(d), rng.standard_normal(d), rng.standard_normal(d)
    kc, ks, vc, vs = oracle.kv_encode(k, v, sg, fmt)
    out = oracle.attend_head(q, kc[None], ks[None], vc[None], vs[None], sg, fmt=fmt)
    if fmt == 1:
        want = brute.dequant_i8(vc, vs)
        assert np.abs(kc).max() <= 7 and np.abs(vc).max() <= 7
        assert np.array_equal(vc, brute.quant(v.astype(np.float32), 7)[0])
    else:
        want = oracle.rht_inverse(brute.dequant_lm(vc, vs), sg)
        assert vc.min() >= 0 and vc.max() <= 7
    assert np.allclose(out, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("fmt", [1, 2])
def test_identical_keys_average_the_values(fmt):
    rng = np.random.default_rng(7)
    d, n = 64, 5
    sg = synth.signs(d, seed=2, stream=11)
    k = rng.standard_normal(d)
    recs = [oracle.kv_encode(k, rng.standard_normal(d), sg, fmt) for _ in range(n)]
    kc, ks, vc, vs = (np.stack([r[i] for r in recs]) for i in range(4))
    out = oracle.attend_head(rng.standard_normal(d), kc, ks, vc, vs, sg, fmt=fmt)
    deq = brute.dequant_i8(vc, vs) if fmt == 1 else brute.dequant_lm(vc, vs)
    mean = deq.mean(0)
    want = mean if fmt == 1 else oracle.rht_inverse(mean, sg)
    assert np.allclose(out, want, rtol=0, atol=1e-12)


# ------------------------------------------------------------- whole model vs brute force
@pytest.mark.parametrize("fmt", [1, 2])
def test_model_with_cache_format_matches_brute_force(fmt):
    shape = W.with_(TINY, kv_format=fmt)
    lw = logical_weights(shape, seed=13, norm_jitter=0.1)
    om = oracle_from_logical(shape, lw)
    bm = brute.BruteModel(shape, lw)
    toks = synth.tokens(6, shape.vocab, seed=13)
    tok = int(toks[0])
    for step in range(16):
        t = int(toks[step]) if step < len(toks) else tok
        xo, lo, ao = om.decode_token(t)
        xb, lb, ab = bm.decode_token(t)
        assert rel_l2(xo, xb) < 1e-10, step
        assert rel_l2(lo, lb) < 1e-10, step
        assert ao == ab
        tok = ao
    for l, t in enumerate(shape.pattern):
        if t == "A":
            kc, ks, vc, vs = om.get_kv(l, om.pos)
            assert np.array_equal(kc, np.stack([e[0] for e in bm.kv[l]]))
            assert np.array_equal(vc, np.stack([e[2] for e in bm.kv[l]]))
            assert np.array_equal(vs, np.stack([e[3] for e in bm.kv[l]]))


def test_formats_differ_and_refuse_window_and_draft():
    """the three formats give three different caches; the variants refuse a
    recent window and a draft head"""
    outs = []
    for fmt in (0, 1, 2):
        shape = W.with_(TINY, kv_format=fmt)
        om = oracle.from_recipe(shape, 2)
        for t in synth.tokens(4, shape.vocab, 2):
            x, _, _ = om.decode_token(int(t))
        outs.append(x)
    assert rel_l2(outs[1], outs[0]) > 1e-6 and rel_l2(outs[2], outs[0]) > 1e-6
    for kw in (dict(kv_window=4), dict(draft_vocab=40)):
        with pytest.raises(MemoryError):
            oracle.Model(W.with_(TINY, kv_format=1, **kw))

"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test names what fixes the expected value: a published known-answer
vector, a library routine, a closed form, an invariant of the mathematics, a
hand-worked case in tests/golden/hand_worked.json, or the independent numpy
brute-force model in oracle/brute.py.
"""
import json
import os

import numpy as np
import pytest
from scipy.linalg import hadamard
from scipy.special import softmax, expit

import oracle
import synth
from oracle import brute
from oracle.accept import accept, inverse_cdf, softmax_t
from tests.helpers import TINY, logical_weights, oracle_from_logical, rel_l2

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")))


# ------------------------------------------------------------- input generator
def test_philox_known_answers():
    # Random123 known-answer vectors for philox4x32-10 (Salmon et al., SC'11)
    assert [hex(v) for v in synth.philox([0, 0, 0, 0], [0, 0])] == \
        ["0x6627e8d5", "0xe169c58d", "0xbc57ac4c", "0x9b00dbd8"]
    assert [hex(v) for v in synth.philox([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2)] == \
        ["0x408f276d", "0x41c83b0e", "0xa20bc7c6", "0x6d5451fd"]
    assert [hex(v) for v in synth.philox([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344],
                                         [0xA4093822, 0x299F31D0])] == \
        ["0xd16cfe09", "0x94fdcceb", "0x5001e420", "0x24126ea1"]


def test_normal_moments():
    z = synth.normal(500, 1000, 1.0, seed=3, stream=9).ravel().astype(np.float64)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    # sigma * z is one fp32 multiply of an exact value
    z2 = synth.normal(500, 1000, 0.02, seed=3, stream=9).ravel()
    assert np.array_equal(z2, (z.astype(np.float32) * np.float32(0.02)).astype(np.float32))


# ------------------------------------------------------------- fp16 and codec
def test_fp16_matches_numpy_cast():
    rng = np.random.default_rng(0)
    vals = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-9, 6, 20000),
                           np.array([0.0, -0.0, 65504, 65519.99, 65520, 1e9, 2 ** -24, 2 ** -25,
                                     3 * 2 ** -26, 2 ** -14, 2 ** -14 - 2 ** -25, 6.1e-5,
                                     np.inf, -np.inf], np.float32)])
    vals = vals.astype(np.float32)
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    ours = oracle.f32_to_f16_bits(vals)
    assert np.array_equal(ours, ref)
    back = oracle.f16_bits_to_f64(ref)
    assert np.array_equal(back, ref.view(np.float16).astype(np.float64))


@pytest.mark.parametrize("case", GOLD["codec"], ids=lambda c: c["name"])
def test_codec_hand_worked(case):
    x = np.zeros(32, np.float32)
    x[:len(case["x"])] = case["x"]
    s, c = oracle.quant_group(x, case["qmax"])
    assert s == case["scale_bits"]
    assert list(c[:len(case["codes"])]) == case["codes"]
    assert not c[len(case["codes"]):].any()


@pytest.mark.parametrize("qmax", [3, 7, 127])
def test_codec_round_trip_exact(qmax):
    rng = np.random.default_rng(qmax)
    for _ in range(200):
        # magnitudes that keep the scale a normal fp16 number (>= 2^-14): there the
        # scale's relative rounding error is at most 2^-11 and amax maps to qmax
        x = (rng.standard_normal(32) * 10.0 ** rng.uniform(-2, 3)).astype(np.float32)
        s, c = oracle.quant_group(x, qmax)
        deq = (c.astype(np.float64) * oracle.f16_bits_to_f64(np.array([s]))[0]).astype(np.float32)
        s2, c2 = oracle.quant_group(deq, qmax)
        assert s2 == s and np.array_equal(c2, c)
        assert np.abs(c).max() <= qmax
        # the largest magnitude lands on +-qmax
        assert np.abs(c).max() == qmax


def test_codec_brute_agrees():
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    for qmax in (3, 7, 127):
        cs, ss = [], []
        for r in range(64):
            for g in range(8):
                s, c = oracle.quant_group(w[r, 32 * g:32 * g + 32], qmax)
                cs.append(c)
                ss.append(s)
        bc, bs = brute.quant(w, qmax)
        assert np.array_equal(np.concatenate(cs), bc.ravel())
        assert np.array_equal(np.array(ss, np.uint16), bs.ravel())


def _pack_nibbles_by_hand(c):
    """logical W4 bytes of integer codes [rows][K]: element 2i in the low
    nibble of byte i, element 2i+1 in the high nibble, nibble = code + 8"""
    out = np.zeros((c.shape[0], c.shape[1] // 2), np.uint8)
    for r in range(c.shape[0]):
        for i in range(c.shape[1] // 2):
            out[r, i] = ((int(c[r, 2 * i]) + 8) & 15) | (((int(c[r, 2 * i + 1]) + 8) & 15) << 4)
    return out


def test_row_quantisers_index_every_slot():
    """oracle.quant_w4 / quant_i8 on a 48 x 256 matrix (8 groups per row) equal
    numpy's group reshape of the same matrix (brute.quant) packed by hand, slot
    by slot.  Every (row, group) gets its own magnitude, so a scale or a code
    written at another (row, group) slot changes a value and fails."""
    rng = np.random.default_rng(7)
    rows, cols = 48, 256
    G = cols // 32
    mag = (1.0 + np.arange(rows * G, dtype=np.float64)).reshape(rows, G) * 1e-3
    w = rng.uniform(-0.9, 0.9, (rows, cols)) * np.repeat(mag, 32, axis=1)
    # one element of each group at +-mag: that group's amax, so its scale is known
    peak = rng.integers(0, 32, (rows, G))
    for r in range(rows):
        for g in range(G):
            w[r, 32 * g + peak[r, g]] = mag[r, g] * (1 if (r + g) % 2 else -1)
    w = w.astype(np.float32)
    # every scale distinct: the slot of each one is checked, not just its value
    bc7, bs7 = brute.quant(w, 7)
    assert len(np.unique(bs7)) == rows * G
    codes, scales = oracle.quant_w4(w)
    assert scales.shape == (rows, G) and codes.shape == (rows, cols // 2)
    assert np.array_equal(scales, bs7)
    assert np.array_equal(codes, _pack_nibbles_by_hand(bc7))
    # the packed codes read back (brute dequant) within half a step of the input
    deq = brute.dequant_w4(codes, scales)
    step = np.repeat(brute.f16(bs7), 32, axis=1)
    assert np.all(np.abs(deq - w) <= 0.5 * step * (1 + 1e-6) + 1e-12)
    bc127, bs127 = brute.quant(w, 127)
    c8, s8 = oracle.quant_i8(w)
    assert np.array_equal(s8, bs127) and np.array_equal(c8, bc127)
    assert np.all(np.abs(brute.dequant_i8(c8, s8) - w) <= 0.5 * np.repeat(brute.f16(bs127), 32, axis=1) * (1 + 1e-6))
    # a transposed operand (rows and groups swapped) is not what the oracle wrote
    assert not np.array_equal(oracle.quant_w4(np.ascontiguousarray(w[::-1]))[1], bs7)


def test_w4_packing_hand_worked():
    g = GOLD["w4_packing"]
    codes = np.zeros(32, np.int64)
    codes[:6] = g["codes"]
    w = (codes * 0.5).astype(np.float32)[None, :]     # amax 3.5 -> scale exactly 0.5
    packed, scales = oracle.quant_w4(w)
    assert list(packed[0, :3]) == g["bytes"]
    assert scales[0, 0] == 0x3800
    assert np.array_equal(brute.dequant_w4(packed, scales)[0], codes * 0.5)


# ------------------------------------------------------------- rotation
def test_rht_hand_worked_and_scipy():
    g = GOLD["rht_d4"]
    assert np.array_equal(oracle.rht_forward(g["v"], g["signs"]), np.array(g["forward"], float))
    rng = np.random.default_rng(2)
    for d in (64, 256):
        s = synth.signs(d, seed=5, stream=11)
        v = rng.integers(-50, 50, d).astype(np.float64)
        ref = hadamard(d) @ (s * v) / np.sqrt(d)
        f = oracle.rht_forward(v, s)
        assert np.allclose(f, ref, rtol=0, atol=1e-12)
        # 1/sqrt(d) is a power of two for d = 64, 256: the round trip is exact
        assert np.array_equal(oracle.rht_inverse(f, s), v)
        assert abs(np.linalg.norm(f) - np.linalg.norm(v)) < 1e-9


# ------------------------------------------------------------- Gated DeltaNet
def test_gdn_hand_worked():
    g = GOLD["gdn_d2"]
    S, o = oracle.gdn_head_step(g["S0"], g["k"], g["v"], g["q"], g["alpha"], g["beta"])
    assert np.array_equal(S, np.array(g["S1"], float))
    assert np.array_equal(o, np.array(g["o"], float))


def test_gdn_invariants():
    rng = np.random.default_rng(3)
    d = 16
    S0 = rng.standard_normal((d, d))
    k = rng.standard_normal(d)
    k /= np.linalg.norm(k)
    v, q = rng.standard_normal(d), rng.standard_normal(d)
    # alpha = 1, beta = 0: state unchanged, o = S q
    S, o = oracle.gdn_head_step(S0, k, v, q, 1.0, 0.0)
    assert np.array_equal(S, S0)
    assert np.allclose(o, S0 @ q, atol=1e-12)
    # beta = 1, |k| = 1: the delta rule writes v at key k, S_t k = v for any alpha
    for alpha in (1.0, 0.7, 0.0):
        S, _ = oracle.gdn_head_step(S0, k, v, q, alpha, 1.0)
        assert np.allclose(S @ k, v, atol=1e-12)
    # alpha = 0: S = beta v k^T
    S, _ = oracle.gdn_head_step(S0, k, v, q, 0.0, 0.3)
    assert np.allclose(S, 0.3 * np.outer(v, k), atol=1e-15)


def test_gdn_expanded_equals_literal_matrix_form():
    rng = np.random.default_rng(4)
    for d in (2, 5, 8):
        S0 = rng.standard_normal((d, d))
        k, v, q = rng.standard_normal(d), rng.standard_normal(d), rng.standard_normal(d)
        a, b = rng.uniform(), rng.uniform()
        S, o = oracle.gdn_head_step(S0, k, v, q, a, b)
        lit = a * S0 @ (np.eye(d) - b * np.outer(k, k)) + b * np.outer(v, k)
        assert np.allclose(S, lit, atol=1e-12)
        assert np.allclose(o, lit @ q, atol=1e-12)


def test_gdn_state_bounded_over_long_run():
    # with unit keys and alpha, beta in (0, 1) every factor alpha (I - beta k k^T) is
    # non-expansive, so |S| stays bounded by sum of beta |v| alpha^j
    rng = np.random.default_rng(5)
    d = 32
    S = np.zeros((d, d))
    peak = 0
    for _ in range(4096):
        k = rng.standard_normal(d)
        k /= np.linalg.norm(k)
        v = rng.standard_normal(d) * 1.4
        a, b = expit(rng.normal(2, 0.5)), expit(rng.normal())
        S, _ = oracle.gdn_head_step(S, k, v, k, a, b)
        peak = max(peak, np.linalg.norm(S))
    assert np.isfinite(peak) and peak < 1.4 * np.sqrt(d) / (1 - expit(3.5)) * 2


# ------------------------------------------------------------- attention
def _rand_cache(rng, npos, d):
    kc = rng.integers(-127, 128, (npos, d)).astype(np.int8)
    vc = rng.integers(-3, 4, (npos, d)).astype(np.int8)
    ks = np.full((npos, d // 32), 0x2000, np.uint16)  # 2^-7
    vs = np.full((npos, d // 32), 0x3400, np.uint16)  # 0.25
    return kc, ks, vc, vs


def test_attention_single_position_returns_its_value():
    rng = np.random.default_rng(6)
    d = 64
    s = synth.signs(d, 1, 11)
    kc, ks, vc, vs = _rand_cache(rng, 1, d)
    out = oracle.attend_head(rng.standard_normal(d), kc, ks, vc, vs, s)
    ref = s * (hadamard(d) @ (vc[0] * 0.25)) / np.sqrt(d)
    assert np.allclose(out, ref, atol=1e-12)


def test_attention_identical_keys_average_values():
    rng = np.random.default_rng(7)
    d, T = 64, 9
    s = synth.signs(d, 2, 11)
    kc, ks, vc, vs = _rand_cache(rng, T, d)
    kc[:] = kc[0]
    out = oracle.attend_head(rng.standard_normal(d) * 3, kc, ks, vc, vs, s)
    ref = s * (hadamard(d) @ (vc.mean(0) * 0.25)) / np.sqrt(d)
    assert np.allclose(out, ref, atol=1e-12)


def test_attention_matches_scipy_softmax():
    rng = np.random.default_rng(8)
    d, T = 64, 37
    s = synth.signs(d, 3, 11)
    kc, ks, vc, vs = _rand_cache(rng, T, d)
    q = rng.standard_normal(d)
    out = oracle.attend_head(q, kc, ks, vc, vs, s)
    p = softmax((kc * 2.0 ** -7) @ q / np.sqrt(d))
    ref = s * (hadamard(d) @ (p @ (vc * 0.25))) / np.sqrt(d)
    assert np.allclose(out, ref, atol=1e-12)


def test_kv_encode_round_trip():
    rng = np.random.default_rng(9)
    d = 256
    s = synth.signs(d, 4, 11)
    k, v = rng.standard_normal(d) * 1.4, rng.standard_normal(d) * 1.4
    kc, ks, vc, vs = oracle.kv_encode(k, v, s)
    kd = kc * np.repeat(oracle.f16_bits_to_f64(ks), 32)
    assert np.max(np.abs(kd - k)) <= np.max(np.abs(k)) / 127 * 0.51
    vr = oracle.rht_forward(v, s)
    vd = vc * np.repeat(oracle.f16_bits_to_f64(vs), 32)
    assert np.abs(vc).max() <= 3
    assert np.max(np.abs(vd - vr)) <= np.max(np.abs(vr)) / 3 * 0.51
    # codes equal the brute codec applied to the fp32 values
    bk, bks = brute.quant(k.astype(np.float32), 127)
    bv, bvs = brute.quant(vr.astype(np.float32), 3)
    assert np.array_equal(bk, kc) and np.array_equal(bks, ks)
    assert np.array_equal(bv, vc) and np.array_equal(bvs, vs)


# ------------------------------------------------------------- whole model vs brute force
@pytest.mark.parametrize("jitter", [0.0, 0.2])
def test_model_matches_brute_force(jitter):
    lw = logical_weights(TINY, seed=11, norm_jitter=jitter)
    om = oracle_from_logical(TINY, lw)
    bm = brute.BruteModel(TINY, lw)
    toks = synth.tokens(6, TINY.vocab, seed=11)
    tok = int(toks[0])
    for step in range(16):
        t = int(toks[step]) if step < len(toks) else tok
        xo, lo, ao = om.decode_token(t)
        xb, lb, ab = bm.decode_token(t)
        assert rel_l2(xo, xb) < 1e-10, step
        assert rel_l2(lo, lb) < 1e-10, step
        assert ao == ab
        tok = ao
    for l, t in enumerate(TINY.pattern):
        if t == "G":
            assert rel_l2(om.get_gdn_state(l), bm.S[l]) < 1e-10
        else:
            kc, ks, vc, vs = om.get_kv(l, om.pos)
            assert np.array_equal(kc, np.stack([e[0] for e in bm.kv[l]]))
            assert np.array_equal(vc, np.stack([e[2] for e in bm.kv[l]]))


def test_argmax_ties_take_lowest_index():
    lw = logical_weights(TINY, seed=12)
    codes, scales = lw[(-1, 5)]
    codes, scales = codes.copy(), scales.copy()
    # make row 100 the unique best, then copy it into rows 7 and 90
    om = oracle_from_logical(TINY, lw)
    x = om.embed(3)
    _, best = om.head(x)
    codes[7], scales[7] = codes[best], scales[best]
    codes[90], scales[90] = codes[best], scales[best]
    om.load_i8(codes, scales)
    logits, am = om.head(x)
    assert logits[7] == logits[best] and am == min(7, best)


# ------------------------------------------------------------- acceptance rule
def test_accept_preserves_target_distribution_chi2():
    from scipy.stats import chisquare
    rng = np.random.default_rng(13)
    V = 8
    p = rng.dirichlet(np.ones(V))
    q = rng.dirichlet(np.ones(V))
    logits = np.log(p)[None, :].repeat(2, 0)
    n = 20000
    u = synth.uniform(2 * n, seed=13, stream=3).reshape(n, 2)
    dr = synth.uniform(n, seed=14, stream=3)
    counts = np.zeros(V)
    for i in range(n):
        d = inverse_cdf(q, dr[i])
        out, _ = accept(logits, [d], q[None, :], u[i], 1.0)
        counts[out[0]] += 1
    stat = chisquare(counts, p * n)
    assert stat.pvalue > 1e-3, stat


def test_accept_chain_marginals():
    # three positions with different fixed targets: each emitted position follows p_j
    from scipy.stats import chisquare
    rng = np.random.default_rng(14)
    V, k = 6, 3
    ps = [rng.dirichlet(np.ones(V)) for _ in range(k + 1)]
    qs = [rng.dirichlet(np.ones(V)) for _ in range(k)]
    logits = np.log(np.stack(ps))
    n = 12000
    u = synth.uniform((k + 1) * n, seed=15, stream=3).reshape(n, k + 1)
    dr = synth.uniform(k * n, seed=16, stream=3).reshape(n, k)
    counts = [np.zeros(V) for _ in range(k + 1)]
    for i in range(n):
        drafts = [inverse_cdf(qs[j], dr[i, j]) for j in range(k)]
        out, _ = accept(logits, drafts, np.stack(qs), u[i], 1.0)
        for j, t in enumerate(out):
            counts[j][t] += 1
    # position 0 is always emitted; later positions are conditioned on reaching them,
    # which with fixed per-position targets still leaves the marginal p_j
    for j in range(k + 1):
        if counts[j].sum() > 500:
            assert chisquare(counts[j], ps[j] * counts[j].sum()).pvalue > 1e-3, j


def test_accept_special_cases():
    V = 10
    rng = np.random.default_rng(15)
    L = rng.standard_normal((4, V))
    # q = p: always accepted
    q = np.stack([softmax_t(L[j], 1.0) for j in range(3)])
    drafts = [3, 1, 4]
    out, na = accept(L, drafts, q, [0.999999, 0.999999, 0.999999, 0.5], 1.0)
    assert na == 3 and out[:3] == drafts and len(out) == 4
    # p(d) = 0 (logit -inf): always rejected, correction drawn from max(0, p - q)
    L2 = L.copy()
    L2[0, 3] = -np.inf
    out, na = accept(L2, drafts, q, [0.0, 0.0, 0.0, 0.5], 1.0)
    assert na == 0 and out[0] != 3 and len(out) == 1
    # temperature 0: exact-match rule, equal to plain greedy
    g = [int(np.argmax(L[j])) for j in range(4)]
    out, na = accept(L, [g[0], g[1], (g[2] + 1) % V], q, [0.5] * 4, 0)
    assert out == [g[0], g[1], g[2]] and na == 2
    out, na = accept(L, g[:3], q, [0.5] * 4, 0)
    assert out == g and na == 3


def test_inverse_cdf_index_order():
    w = np.array([0.0, 0.25, 0.0, 0.5, 0.25])
    assert inverse_cdf(w, 0.0) == 1
    assert inverse_cdf(w, 0.2499) == 1
    assert inverse_cdf(w, 0.25) == 3
    assert inverse_cdf(w, 0.7499) == 3
    assert inverse_cdf(w, 0.75) == 4
    assert inverse_cdf(w, 0.9999) == 4


@pytest.mark.parametrize("wrong", [None, 0, 2])
def test_verify_commit_equals_decoding_the_accepted_prefix(wrong):
    """A verify pass commits what decoding the accepted prefix one token at a
    time gives (the acceptance rule keeps the target's own tokens; the rejected
    drafts leave no trace): from the same state, the position, every GDN
    state, every cache entry and the next token's logits equal those of a model
    that decoded t0 .. d_a alone.  Greedy drafts with none, the first or the
    third made wrong (a = 3, 0, 2)."""
    from oracle.accept import verify
    from tests.helpers import TINY, logical_weights, oracle_from_logical
    lw = logical_weights(TINY, seed=31, norm_jitter=0.1)
    om, ref = oracle_from_logical(TINY, lw), oracle_from_logical(TINY, lw)
    prompt = synth.tokens(9, TINY.vocab, 31)
    for t in prompt[:-1]:
        om.decode_token(int(t))
        ref.decode_token(int(t))
    t0 = int(prompt[-1])
    snap = om.snapshot()
    chain, t = [], t0
    for _ in range(3):
        _, _, t = om.decode_token(t)
        chain.append(int(t))
    om.restore(snap)
    if wrong is not None:
        chain[wrong] = (chain[wrong] + 1) % TINY.vocab
    out, a, _ = verify(om, [t0] + chain, None, None, 0.0)
    assert a == (3 if wrong is None else wrong)
    for t in [t0] + chain[:a]:
        ref.decode_token(t)
    assert om.pos == ref.pos
    for l, kind in enumerate(TINY.pattern):
        if kind == "G":
            assert np.array_equal(om.get_gdn_state(l), ref.get_gdn_state(l)), l
        else:
            for x, y in zip(om.get_kv(l, om.pos), ref.get_kv(l, ref.pos)):
                assert np.array_equal(x, y), l
    _, L1, _ = om.decode_token(out[-1])
    _, L2, _ = ref.decode_token(out[-1])
    assert np.array_equal(L1, L2)

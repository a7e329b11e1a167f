"""Pins of the oracle's draft head (no GPU needed).

What fixes each expected value: the independent numpy model in oracle/brute.py
(test_draft_step_matches_brute_force), a closed form of the input combination
(one-hot fuse rows with the draft block's output projections zeroed), the
oracle's own full output head restricted to the mapped ids, the definition of
the map as a set of ids, and a chi-square test of the draws against q.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import brute
from oracle.draft import DraftDriver, select
from synth import workloads as W
from tests.helpers import TINY_MTP, logical_weights, oracle_from_logical, rel_l2

D = TINY_MTP.n_layers
H = TINY_MTP.hidden


def _models(seed=21, jitter=0.2):
    lw = logical_weights(TINY_MTP, seed=seed, norm_jitter=jitter)
    return lw, oracle_from_logical(TINY_MTP, lw), brute.BruteModel(TINY_MTP, lw)


def test_draft_step_matches_brute_force():
    lw, om, bm = _models()
    rng = np.random.default_rng(3)
    toks = synth.tokens(12, TINY_MTP.vocab, seed=21)
    h = rng.standard_normal(H)
    # committed entries, then speculative ones at growing slots, then more commits
    for i, t in enumerate(toks):
        slot = 0 if i % 4 == 0 else (i % 4) - 1
        xo, zo = om.draft_step(int(t), h, slot)
        bm.dpos = om.dpos
        xb, zb = bm.draft_step(int(t), h, slot)
        assert rel_l2(xo, xb) < 1e-10, i
        assert rel_l2(zo, zb) < 1e-10, i
        if i % 4 == 0:
            om.set_dpos(om.dpos + 1)
        h = xo
    kc, ks, vc, vs = om.get_kv(D, om.dpos + 2)
    assert np.array_equal(kc, np.stack([e[0] for e in bm.kv[D][:om.dpos + 2]]))
    assert np.array_equal(vc, np.stack([e[2] for e in bm.kv[D][:om.dpos + 2]]))


def test_draft_fuse_one_hot_closed_form():
    """Fuse rows that copy one input column each (code 1, scale 1.0) and a draft
    block whose output projections are zero: the step's output is the selected
    entries of [fp16(norm_e(embedding)); fp16(norm_h(h))] exactly."""
    lw, om, _ = _models(seed=22)
    rng = np.random.default_rng(4)
    cols = rng.integers(0, 2 * H, H)
    nib = np.full((H, 2 * H), 8, np.uint8)
    nib[np.arange(H), cols] = 9
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = np.zeros((H, 2 * H // 32), np.uint16)
    scales[np.arange(H), cols // 32] = 0x3C00
    om.load_w4(D, W.T_DRAFT_FUSE, codes, scales)
    for kind in (W.T_MIX_OUT, W.T_FFN_DOWN):
        c, s = lw[(D, kind)]
        om.load_w4(D, kind, np.full_like(c, 0x88), np.zeros_like(s))
    token = 77
    h = rng.standard_normal(H) * 3.0
    x, _ = om.draft_step(token, h, 0)
    ec, es = lw[(-1, W.T_LM_HEAD)]
    e = ec[token].astype(np.float64) * np.repeat(es[token].view(np.float16).astype(np.float64), 32)
    eps = TINY_MTP.rms_eps

    def norm(v, w):
        return v / np.sqrt(np.mean(v * v) + eps) * w

    u = np.concatenate([norm(e, lw[(D, W.T_DRAFT_NORM_EMB)]), norm(h, lw[(D, W.T_DRAFT_NORM_HID)])])
    u = u.astype(np.float32).astype(np.float16).astype(np.float64)
    assert np.array_equal(x, u[cols])


def test_draft_scores_equal_full_head_on_mapped_ids():
    lw, om, _ = _models(seed=23)
    om.load_vec(D, W.T_DRAFT_NORM_OUT, lw[(-1, W.T_NORM_FINAL)].astype(np.float32))
    x, z = om.draft_step(5, np.ones(H), 0)
    full, _ = om.head(x)
    ids = om.draft_map()
    assert np.array_equal(ids, np.sort(lw[(D, W.T_DRAFT_MAP)]))
    assert rel_l2(z, full[ids]) < 1e-14


def test_draft_map_order_and_validation():
    lw, om, _ = _models(seed=24)
    ids = lw[(D, W.T_DRAFT_MAP)]
    x0, z0 = om.draft_step(9, np.ones(H), 0)
    om.set_draft_map(np.random.default_rng(5).permutation(ids))
    assert np.array_equal(om.draft_map(), np.sort(ids))
    x1, z1 = om.draft_step(9, np.ones(H), 0)
    assert np.array_equal(z0, z1)
    bad = ids.copy()
    bad[1] = bad[0]
    with pytest.raises(ValueError):
        om.set_draft_map(bad)
    bad = ids.copy()
    bad[0] = TINY_MTP.vocab
    with pytest.raises(ValueError):
        om.set_draft_map(bad)
    with pytest.raises(ValueError):
        om.set_draft_map(ids[:-1])


def test_draft_map_recipe_is_a_uniform_subset():
    s = W.with_(TINY_MTP, vocab=4096, draft_vocab=1024)
    ids = synth.draft_map(s, 0)
    assert len(ids) == 1024 and len(np.unique(ids)) == 1024
    assert ids.min() >= 0 and ids.max() < 4096 and np.all(np.diff(ids) > 0)
    # about a quarter of every quarter of the id range
    counts = np.histogram(ids, bins=4, range=(0, 4096))[0]
    assert np.all(np.abs(counts - 256) < 60)


def test_select_greedy_ties_take_lowest_id():
    lw, om, _ = _models(seed=25)
    x, z = om.draft_step(3, np.ones(H), 0)
    ids = om.draft_map()
    best = int(np.argmax(z))
    # copy the best mapped row into an earlier and a later mapped row
    codes, scales = (a.copy() for a in lw[(-1, W.T_LM_HEAD)])
    for j in (best // 2, min(best + 3, len(ids) - 1)):
        codes[ids[j]], scales[ids[j]] = codes[ids[best]], scales[ids[best]]
    om.load_i8(codes, scales)
    x2, z2 = om.draft_step(3, np.ones(H), 0)
    i, q = select(z2, 0.0, None)
    assert q is None and i == min(best // 2, best) and z2[i] == z2.max()


def test_select_draws_follow_q_chi2():
    from scipy.stats import chisquare
    rng = np.random.default_rng(6)
    z = rng.standard_normal(12) * 1.5
    T = 0.8
    n = 200000
    counts = np.zeros(12)
    for u in rng.random(n):
        i, q = select(z, T, u)
        counts[i] += 1
    e = np.exp(z / T - (z / T).max())
    p = e / e.sum()
    assert np.allclose(q, p, rtol=1e-12)
    assert chisquare(counts, p * n).pvalue > 1e-3


def test_speculative_entries_are_not_committed():
    """Drafting k = 3 then verifying gives the same draft-head cache and the
    same next drafts as drafting k = 1 before the same verify."""
    lw = logical_weights(TINY_MTP, seed=26, norm_jitter=0.1)
    prompt = synth.tokens(6, TINY_MTP.vocab, seed=26)
    runs = []
    for k in (3, 1):
        dd = DraftDriver(oracle_from_logical(TINY_MTP, lw))
        _, _, am = dd.prefill(prompt)
        d, _, _ = dd.draft(am, k)
        out, a, _ = dd.verify([am] + [7, 8, 9], None, None, 0.0)
        d2, _, z2 = dd.draft(out[-1], 3)
        runs.append((dd.m.dpos, d2, z2, dd.m.get_kv(D, dd.m.dpos)))
    assert runs[0][0] == runs[1][0] == len(prompt) + 1
    assert runs[0][1] == runs[1][1] and np.array_equal(runs[0][2], runs[1][2])
    for a, b in zip(runs[0][3], runs[1][3]):
        assert np.array_equal(a, b)


def test_speculative_greedy_equals_plain_greedy():
    lw = logical_weights(TINY_MTP, seed=27, norm_jitter=0.1)
    prompt = synth.tokens(5, TINY_MTP.vocab, seed=27)
    ref = oracle_from_logical(TINY_MTP, lw)
    for t in prompt:
        _, _, am = ref.decode_token(int(t))
    plain = [am]
    for _ in range(12):
        _, _, am = ref.decode_token(plain[-1])
        plain.append(am)
    dd = DraftDriver(oracle_from_logical(TINY_MTP, lw))
    _, _, t0 = dd.prefill(prompt)
    got = [t0]
    accepted = 0
    while len(got) < len(plain):
        drafts, _, _ = dd.draft(got[-1], 3)
        # every other pass checks the target's own greedy tokens so that long
        # accepted runs (and their pending draft-head entries) occur
        if len(got) % 2:
            drafts = plain[len(got):len(got) + 3] + [0] * max(0, len(got) + 3 - len(plain))
        out, a, _ = dd.verify([got[-1]] + drafts[:3], None, None, 0.0)
        accepted += a
        got.extend(out)
    assert got[:len(plain)] == plain
    assert accepted >= 3

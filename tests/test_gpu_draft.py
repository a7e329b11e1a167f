"""GPU parity of the draft head (aw4_draft) against the oracle.

The oracle side is oracle/draft.py's DraftDriver on an oracle model built from
the same seeded recipe: it feeds the draft head's cache in the order the
library does (prompt positions during prefill, positions accepted by a verify
pass at the next draft call) and runs or_draft_step for every entry.  Passes
start from the oracle's imported state (teacher forcing: a cached code at a
rounding tie moves the target's hidden state by a few percent, see the parity
methodology), on the toy stack with a 1,024-id map; mapped scores must agree
to 1e-2 relative L2; greedy drafts, verify results and cache lengths must be
identical; new draft-cache codes may differ only by one at rounding ties.
Some passes verify the target's own greedy continuation instead of the
drafts, so that all three drafts are accepted and the next draft call feeds
four entries in one pass.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from oracle.accept import inverse_cdf, softmax_t
from oracle.draft import DraftDriver
from synth import state as SS
from synth import workloads as W
from tests.helpers import rel_l2

pytestmark = pytest.mark.gpu

SHAPE = W.TOY_MTP
D = SHAPE.n_layers


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


def _pair(A, seed, jitter=0.1):
    from synth.gpu_load import load_recipe
    om = oracle.from_recipe(SHAPE, seed, jitter)
    gm = A.Model(SHAPE)
    load_recipe(gm, SHAPE, seed, jitter)
    return DraftDriver(om), gm


def _greedy_chain(om, t0, n):
    snap = om.snapshot()
    out, t = [], t0
    for _ in range(n):
        _, _, t = om.decode_token(t)
        out.append(t)
    om.restore(snap)
    return out


def test_draft_weights_bit_exact(aw4):
    _say("case: draft head weights, toy stack, seed 5")
    dd, gm = _pair(aw4, 5)
    from tests.helpers import logical_weights
    lw = logical_weights(SHAPE, 5, 0.1)
    for kind in (W.T_DRAFT_FUSE, W.T_MIX_IN, W.T_FFN_DOWN):
        c, s = gm.export_tensor(D, kind)
        assert np.array_equal(c, lw[(D, kind)][0]) and np.array_equal(s, lw[(D, kind)][1]), kind
    gm.close()


def _import(gm, om):
    """the oracle's target state and draft cache into the GPU model"""
    for l, t in enumerate(SHAPE.pattern):
        if t == "G":
            gm.import_gdn(l, om.get_gdn_state(l).astype(np.float32))
        else:
            gm.import_kv(l, *om.get_kv(l, om.pos))
    gm.set_pos(om.pos)
    gm.import_kv(D, *om.get_kv(D, om.dpos))
    gm.set_dpos(om.dpos)


def _check_entries(gm, om, e0):
    """draft cache entries e0 .. dpos: codes equal up to rounding ties"""
    n = om.dpos
    assert gm.dpos == n
    gk, ok = gm.export_kv(D, n), om.get_kv(D, n)
    for a, b in ((gk[0], ok[0]), (gk[2], ok[2])):
        d = a[e0:].astype(int) - b[e0:].astype(int)
        assert np.abs(d).max() <= 1 and (d != 0).mean() < 6e-2


def test_draft_greedy_matches_oracle(aw4):
    """Teacher-forced passes: each starts from the oracle's target state and
    draft cache, runs one decode step, a draft call (one entry fed), a verify
    pass of the target's own greedy continuation (all accepted) and a second
    draft call (four entries fed in one pass), then verifies those drafts."""
    import torch
    _say("case: draft head greedy, toy stack, seed 6")
    dd, gm = _pair(aw4, 6)
    om = dd.m
    prompt = synth.tokens(16, SHAPE.vocab, 6)
    # prefill feeds every prompt position but the last
    gm.prefill(prompt[:-1])
    dd.prefill(prompt[:-1])
    assert gm.dpos == om.dpos == len(prompt) - 2
    t = int(prompt[-1])
    scores = torch.empty(3, SHAPE.draft_vocab, dtype=torch.float32, device="cuda")
    accepted = 0
    for p in range(5):
        _import(gm, om)
        e0 = om.dpos
        tg = gm.decode_step(t)
        _, _, t0 = dd.decode(t)
        assert tg == t0, p
        for step in range(2):
            d0 = om.dpos
            got = gm.draft(t0, 3, scores=scores)
            ref, _, z = dd.draft(t0, 3)
            for j in range(3):
                err = rel_l2(scores[j].cpu().numpy(), z[j])
                assert err < 1e-2, (p, step, j, err)
            assert got == ref, (p, step, got, ref)
            assert om.dpos - d0 == (1 if step == 0 else 4)
            _check_entries(gm, om, e0)
            drafts = _greedy_chain(om, t0, 3) if step == 0 else ref
            out_g = gm.verify_k([t0] + drafts, temperature=0.0)
            out_o, a, _ = dd.verify([t0] + drafts, None, None, 0.0)
            assert out_g == out_o, (p, step, out_g, out_o)
            assert gm.pos == om.pos
            accepted += a
            t0 = out_o[-1]
        # next pass: the last emitted token runs through a plain decode step
        t = t0
    _say("accepted drafts", accepted)
    gm.close()


def test_draft_sampling_matches_oracle(aw4):
    """T = 1: q over the whole vocabulary (zero outside the map) against the
    oracle's, and each draw equal to the oracle's inverse-CDF draw unless the
    uniform sits at the oracle's own CDF boundary.  Drafts 2 and 3 are fed the
    GPU's drafts on both sides."""
    import torch
    _say("case: draft head sampling T=1, toy stack, seed 7")
    dd, gm = _pair(aw4, 7)
    prompt = synth.tokens(12, SHAPE.vocab, 7)
    gm.prefill(prompt)
    _, _, t0 = dd.prefill(prompt)
    ids = dd.map
    q = torch.empty(3, SHAPE.vocab, dtype=torch.float32, device="cuda")
    exact = near = 0
    for p in range(6):
        u = synth.uniform(3, 7, W.STREAM_UNIFORM, i0=16 * p)
        got = gm.draft(t0, 3, 1.0, u, q=q)
        ref, qo, _ = dd.draft(t0, 3, 1.0, u, force=got)
        qg = q.cpu().numpy()
        outside = np.ones(SHAPE.vocab, bool)
        outside[ids] = False
        assert np.all(qg[:, outside] == 0.0)
        for j in range(3):
            assert rel_l2(qg[j], qo[j]) < 1e-2, (p, j)
            if got[j] == ref[j]:
                exact += 1
                continue
            c = np.cumsum(qo[j][ids])
            i = int(np.searchsorted(ids, got[j]))
            lo, hi = (c[i - 1] if i else 0.0), c[i]
            assert lo - 1e-3 <= u[j] <= hi + 1e-3, (p, j, got[j], ref[j], u[j], lo, hi)
            near += 1
        out_g = gm.verify_k([t0] + got, q, np.append(u, 0.5).astype(np.float32), 1.0)
        out_o, _, _ = dd.verify([t0] + got, qg.astype(np.float64), np.append(u, 0.5), 1.0)
        if out_g != out_o:
            break   # an acceptance at its boundary; the two sides no longer share a state
        t0 = out_o[-1]
    _say(f"draws equal {exact}, at a boundary {near}")
    assert exact >= 6
    gm.close()


def test_speculative_greedy_equals_plain_greedy(aw4):
    """Drafting with the draft head and verifying at temperature 0 emits exactly
    the tokens of plain greedy decoding (GPU only)."""
    _say("case: speculative greedy vs plain greedy, toy stack, seed 8")
    from synth.gpu_load import load_recipe
    gm = aw4.Model(SHAPE)
    load_recipe(gm, SHAPE, 8, 0.1)
    prompt = synth.tokens(16, SHAPE.vocab, 8)
    gm.prefill(prompt[:-1])
    plain = [int(prompt[-1])] + list(gm.decode_greedy(int(prompt[-1]), 40))
    gm.reset()
    gm.prefill(prompt[:-1])
    gm.decode_step(int(prompt[-1]), want_argmax=False)
    got = [int(prompt[-1])]
    t0 = plain[1]
    got.append(t0)
    while len(got) < len(plain):
        drafts = gm.draft(t0, 3)
        out = gm.verify_k([t0] + drafts, temperature=0.0)
        got.extend(out)
        t0 = out[-1]
    assert got[:len(plain)] == plain
    gm.close()


def test_draft_errors(aw4):
    _say("case: draft head error paths, toy stack")
    from synth.gpu_load import load_recipe
    gm = aw4.Model(SHAPE)
    with pytest.raises(aw4.AW4Error) as e:
        gm.draft(1, 3)
    assert e.value.code == -8          # no map (and no weights) yet
    load_recipe(gm, SHAPE, 0)          # every tensor, the map included
    with pytest.raises(aw4.AW4Error) as e:
        gm.draft(1, 3)
    assert e.value.code == -8          # nothing committed to draft from
    gm.decode_step(3)
    for bad in (dict(k=0), dict(k=4)):
        with pytest.raises(aw4.AW4Error) as e:
            gm.draft(1, bad["k"])
        assert e.value.code == -1
    with pytest.raises(aw4.AW4Error) as e:
        gm.draft(SHAPE.vocab, 3)
    assert e.value.code == -7
    with pytest.raises(aw4.AW4Error) as e:
        gm.draft(1, 3, 1.0, None)
    assert e.value.code == -1          # sampling needs uniforms
    assert len(gm.draft(1, 3)) == 3
    with pytest.raises(aw4.AW4Error) as e:
        gm.draft(1, 3)
    assert e.value.code == -8          # one draft call per committed state
    bad = synth.draft_map(SHAPE, 0)
    bad[3] = bad[2]
    with pytest.raises(aw4.AW4Error):
        gm.set_draft_map(bad)
    gm.close()


def test_draft_from_synthetic_long_cache(aw4):
    """A draft call over a synthetic 900-entry draft cache (and 901-position
    target caches) against the oracle with the same imported state."""
    import torch
    _say("case: draft head over a 900-entry synthetic cache, toy stack, seed 9")
    dd, gm = _pair(aw4, 9)
    SS.fill(gm, SHAPE, 901, 9)
    SS.fill(dd.m, SHAPE, 901, 9)
    assert gm.dpos == dd.m.dpos == 900
    first = int(synth.tokens(1, SHAPE.vocab, 9, i0=901)[0])
    t0 = gm.decode_step(first)
    _, _, t0o = dd.decode(first)
    assert t0 == t0o
    scores = torch.empty(3, SHAPE.draft_vocab, dtype=torch.float32, device="cuda")
    got = gm.draft(t0, 3, scores=scores)
    ref, _, z = dd.draft(t0, 3)
    for j in range(3):
        assert rel_l2(scores[j].cpu().numpy(), z[j]) < 1e-2, j
    assert got == ref and gm.dpos == 901
    gm.close()

"""Full-size parity: the 27B-shape stack (64 layers, vocab 248320) on one
MI355X, in the launch configuration the benchmark times (captured HIP graph per
token, aw4_decode_greedy), against the oracle from the same seeded weights and
the same synthetic 8192-position state.  Greedy tokens must be identical and
the final hidden state within 1e-2 relative L2.  The oracle is slow at this
size (about a second per token on the host cores), so the check covers 24
steps; the smallest top-2 logit margin the oracle sees is reported.  From the
same state, one decode step and three drafts of the draft head (65,536 mapped
ids, an 8191-entry synthetic draft cache) are checked the same way: drafts
identical, mapped scores within 1e-2 relative L2.
"""
import os
import sys
import time

import numpy as np
import pytest

import oracle
import synth
from synth import state as SS
from oracle.draft import DraftDriver
from synth import workloads as W
from tests.helpers import rel_l2

pytestmark = pytest.mark.gpu

CTX = 8192
STEPS = 24
SHAPE = W.with_(W.FULL_27B, max_ctx=CTX + 64)
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "full_27b_greedy_8k.json")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def full_oracle():
    """the oracle of the full stack (draft head included), built once"""
    t0 = time.time()
    om = oracle.from_recipe(SHAPE, 0)
    _say(f"oracle built in {time.time() - t0:.1f} s")
    return om


# Tie bound for the 256-step greedy test.  GEMV inputs are fp16 (A16): the GPU
# rounds fp32 values and the oracle fp64 values, so at a rounding tie one
# activation lands one fp16 ulp apart (a large SwiGLU output: 0.016), which
# moves that layer's output by about 1e-4 relative; over 64 layers of random
# weights these flips hold the final hidden state about 5.5e-3 from the
# oracle's (measured after 32 to 128 teacher-forced steps) and the top-2 logit
# margin within 0.034 of the oracle's (median 0.008, 256 steps).  Where the
# oracle's margin is below MARGIN_TIE the two sides may take either token.
MARGIN_TIE = 0.05
LOGIT_TOL = 0.1


@pytest.mark.timeout(600)
def test_full_27b_greedy_256():
    """256 greedy steps of the full stack from the seeded synthetic
    8192-position state against the oracle's run, stored by
    tests/golden/make_full_greedy.py (oracle only): its tokens, its four
    largest logits per step and its hidden state after steps 32 ... 256.
    Free-running, in the benchmark's launch configuration (one captured graph
    per token, aw4_decode_greedy): tokens identical up to the first step whose
    oracle top-2 margin is below MARGIN_TIE, where the GPU may take the
    runner-up instead.  Teacher-forced on the oracle's tokens (aw4_decode_step
    with logits): the oracle's token wherever its margin is at least
    MARGIN_TIE and else one of its top two, the logits of the oracle's top
    four ids within LOGIT_TOL, the hidden state within 1e-2 relative L2 at
    every stored step."""
    import base64
    import json
    import torch
    import attention_w4_amd as A
    from synth.gpu_load import load_recipe
    gold = json.load(open(GOLDEN))
    n, toks, top = gold["steps"], gold["tokens"], gold["top4"]
    margin = [t[1][0] - t[1][1] for t in top]
    shape = W.with_(W.FULL_27B, max_ctx=gold["ctx"] + n + 8, draft_vocab=0)
    _say(f"case: full 27B-shape stack, {n} greedy steps against the stored oracle run")
    gm = A.Model(shape)
    load_recipe(gm, shape, gold["seed"])
    SS.fill(gm, shape, gold["ctx"], gold["seed"])
    got = [int(t) for t in gm.decode_greedy(gold["first"], n)]
    k = next((i for i in range(n) if got[i] != toks[i]), n)
    _say(f"free-running: identical for {k} steps" + (
        "" if k == n else f"; step {k}: GPU {got[k]}, oracle {toks[k]} (runner-up {top[k][0][1]}), "
                          f"oracle margin {margin[k]:.2e}"))
    assert k == n or (margin[k] < MARGIN_TIE and got[k] == top[k][0][1])
    # teacher-forced: the oracle's tokens in, logits out
    SS.fill(gm, shape, gold["ctx"], gold["seed"])
    lo = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    tok, worst, flips, herr = gold["first"], 0.0, [], {}
    for i in range(n):
        am = gm.decode_step(tok, lo)
        ids, vals = top[i]
        gl = lo[torch.tensor(ids, device="cuda")].cpu().numpy().astype(np.float64)
        worst = max(worst, float(np.abs(gl - np.asarray(vals)).max()))
        if am != toks[i]:
            flips.append(i)
            assert margin[i] < MARGIN_TIE and am == ids[1], (i, am, ids, vals)
        if str(i + 1) in gold["hidden_after"]:
            ref = np.frombuffer(base64.b64decode(gold["hidden_after"][str(i + 1)]), "<f4").astype(np.float64)
            herr[i + 1] = rel_l2(gm.read_hidden(), ref)
        tok = toks[i]
    gm.close()
    del gm
    torch.cuda.empty_cache()
    _say(f"teacher-forced: argmax differs at {flips} (oracle margins "
         f"{[round(margin[i], 5) for i in flips]}); worst top-4 logit difference {worst:.2e}; "
         f"hidden rel-L2 {', '.join(f'{s}: {e:.2e}' for s, e in herr.items())}")
    assert worst < LOGIT_TOL
    assert herr and max(herr.values()) < 1e-2


@pytest.mark.timeout(1200)
def test_full_27b_greedy_from_8k_state(full_oracle):
    import torch
    import attention_w4_amd as A
    from synth.gpu_load import load_recipe
    shape = SHAPE
    _say("case: full 27B-shape stack, 8192-position synthetic state, greedy", STEPS)
    t0 = time.time()
    gm = A.Model(shape)
    load_recipe(gm, shape, 0)
    SS.fill(gm, shape, CTX, 0)
    first = int(synth.tokens(1, shape.vocab, 0, i0=CTX)[0])
    got = gm.decode_greedy(first, STEPS)
    xg = gm.read_hidden()
    # the same state again through one verify pass of three drafts at
    # temperature 0, which runs the multi-token (M = 4) projections at every
    # 27B shape: the greedy drafts are all accepted and the bonus token is the
    # fourth greedy token
    SS.fill(gm, shape, CTX, 0)
    emitted = gm.verify_k([first] + [int(t) for t in got[:3]], temperature=0.0)
    vpos = gm.pos
    # the draft head from the same state: one decode step, then three drafts
    SS.fill(gm, shape, CTX, 0)
    t1 = gm.decode_step(first)
    scores = torch.empty(3, shape.draft_vocab, dtype=torch.float32, device="cuda")
    drafts = gm.draft(t1, 3, scores=scores)
    sc = scores.cpu().numpy()
    # a verify pass of the greedy continuation (all three accepted), then a draft
    # call that feeds its four entries in one pass
    emitted2 = gm.verify_k([t1] + [int(t) for t in got[1:4]], temperature=0.0)
    drafts2 = gm.draft(emitted2[-1], 3, scores=scores)
    sc2 = scores.cpu().numpy()
    gm.close()
    del gm
    torch.cuda.empty_cache()
    _say(f"gpu done in {time.time() - t0:.1f} s")
    om = full_oracle
    SS.fill(om, shape, CTX, 0)
    t0 = time.time()
    dd = DraftDriver(om)
    _, _, t1o = dd.decode(first)
    dref, _, z = dd.draft(t1o, 3)
    derr = [rel_l2(sc[j], z[j]) for j in range(3)]
    out2, _, _ = dd.verify([t1o] + [int(t) for t in got[1:4]], None, None, 0.0)
    dref2, _, z2 = dd.draft(out2[-1], 3)
    derr += [rel_l2(sc2[j], z2[j]) for j in range(3)]
    _say(f"oracle drafts in {time.time() - t0:.1f} s: {dref} then {dref2} (gpu {drafts} then {drafts2}), "
         f"score rel-L2 {derr}")
    SS.fill(om, shape, CTX, 0)
    tok, ref, margins = first, [], []
    t0 = time.time()
    for i in range(STEPS):
        x, lo, tok = om.decode_token(tok)
        s = np.sort(lo)
        margins.append(float(s[-1] - s[-2]))
        ref.append(tok)
    _say(f"oracle {STEPS} steps in {time.time() - t0:.1f} s; smallest top-2 margin {min(margins):.3e}; "
         f"final hidden rel-L2 {rel_l2(xg, x):.2e}")
    _say("gpu   ", list(got))
    _say("oracle", ref)
    _say("verify", emitted, "position", vpos)
    assert list(got) == ref
    assert emitted == ref[:4] and vpos == CTX + 4
    assert t1 == t1o == ref[0] and drafts == dref and max(derr) < 1e-2
    assert emitted2 == out2 == ref[1:5] and drafts2 == dref2
    assert rel_l2(xg, x) < 1e-2


def _import_target(gm, om, shape):
    """the oracle's recurrent states and caches (target layers) and position"""
    for l, t in enumerate(shape.pattern):
        if t == "G":
            gm.import_gdn(l, om.get_gdn_state(l).astype(np.float32))
        else:
            gm.import_kv(l, *om.get_kv(l, om.pos))
    gm.set_pos(om.pos)


def _decision_boundary(got, ref, L, q, drafts, u, k, tol=1e-4):
    """True if the first difference between two verify outcomes sits at the
    oracle's own decision boundary: the uniform within tol of min(1, p/q) for
    an accept/reject decision, or within tol of the cumulative mass at the
    index where the two drawn tokens part for the final draw"""
    from oracle.accept import softmax_t
    for j in range(min(len(got), len(ref))):
        if got[j] == ref[j]:
            continue
        p = softmax_t(L[j], 1.0)
        if j < k:
            thr = min(1.0, p[drafts[j]] / q[j][drafts[j]])
            if abs(u[j] - thr) < tol:
                return True
            if len(got) != len(ref):
                return False     # one side kept draft j, the other did not
            w = np.maximum(p - q[j], 0.0)
            if w.sum() <= 0:
                w = p
        else:
            w = p
        c = np.cumsum(w) / w.sum()
        lo = min(got[j], ref[j])
        return abs(c[lo] - u[k]) < tol
    return False


@pytest.mark.timeout(1200)
def test_full_27b_sampling_verify_and_draft(full_oracle):
    """Draft verification at temperature 1 on the full stack (k = 3, synthetic
    draft distributions q over all 248,320 ids: the acceptance and residual
    draws run over the whole vocabulary, 122 chunks with a ragged last one),
    three passes, each from the oracle's state; then the draft head at
    temperature 1 (q over its 65,536 mapped ids, draws by inverse CDF) from
    the committed positions of the last pass.  Outcomes must equal the
    oracle's except at the oracle's own decision boundary; the draft
    probabilities and mapped scores within 1e-2 relative L2."""
    import torch
    import attention_w4_amd as A
    from oracle.accept import softmax_t, inverse_cdf
    from synth.gpu_load import load_recipe
    shape, k, V = SHAPE, 3, SHAPE.vocab
    _say("case: full stack, T = 1 verify (3 passes) and T = 1 draft head")
    gm = A.Model(shape)
    load_recipe(gm, shape, 0)
    SS.fill(gm, shape, CTX, 0)
    om = full_oracle
    SS.fill(om, shape, CTX, 0)
    dd = DraftDriver(om)
    t0 = int(synth.tokens(1, V, 0, i0=CTX + 7)[0])
    # the first pass's t0 follows the synthetic state directly: decode it on
    # both sides so that both hold a committed hidden state
    g0 = gm.decode_step(t0)
    _, _, r0 = dd.decode(t0)
    assert g0 == r0
    t = r0
    agree = near = 0
    for p in range(3):
        logits = synth.normal(k, V, W.DRAFT_LOGIT_STD, 11, W.STREAM_DRAFT + p).astype(np.float64)
        q = np.stack([softmax_t(logits[j], 1.0) for j in range(k)]).astype(np.float32)
        du = synth.uniform(k, 11, W.STREAM_UNIFORM, i0=4000 + 8 * p)
        drafts = [inverse_cdf(q[j], du[j]) for j in range(k)]
        u = synth.uniform(k + 1, 11, W.STREAM_UNIFORM, i0=5000 + 8 * p)
        _import_target(gm, om, shape)
        got = gm.verify_k([t] + drafts, torch.from_numpy(q).cuda(), u, 1.0)
        ref, a, L = dd.verify([t] + drafts, q.astype(np.float64), u, 1.0)
        _say(f"pass {p}: gpu {got} oracle {ref} (drafts {drafts})")
        if got == ref:
            agree += 1
        else:
            # the same number of drafts kept unless the acceptance itself sat at
            # its boundary; a differing draw within 1e-4 of cumulative mass of u
            # (over 248,320 ids each CDF step is about 4e-6 wide, so fp32
            # probabilities move the drawn index by a few ids)
            assert _decision_boundary(got, ref, L, q.astype(np.float64), drafts, u, k), (p, got, ref)
            near += 1
        t = ref[-1]
    _say(f"passes equal {agree}, differing at a decision boundary {near}")
    # the draft head from the last pass's committed positions (if that pass
    # agreed both sides hold the same pending entries)
    qd = torch.empty(k, V, dtype=torch.float32, device="cuda")
    sd = torch.empty(k, shape.draft_vocab, dtype=torch.float32, device="cuda")
    dus = synth.uniform(k, 12, W.STREAM_UNIFORM, i0=6000)
    gd = gm.draft(t, k, 1.0, dus, q=qd, scores=sd)
    rd, rq, rz = dd.draft(t, k, 1.0, dus, force=gd)
    gq, gz = qd.cpu().numpy(), sd.cpu().numpy()
    qerr = [rel_l2(gq[j], rq[j]) for j in range(k)]
    zerr = [rel_l2(gz[j], rz[j]) for j in range(k)]
    _say(f"draft T=1: gpu {gd} oracle {rd}; q rel-L2 {qerr}; score rel-L2 {zerr}")
    assert max(qerr) < 1e-2 and max(zerr) < 1e-2
    for j in range(k):
        if gd[j] != rd[j]:
            m = om.draft_map()
            c = np.cumsum(rq[j][m]) / rq[j][m].sum()
            lo = int(np.searchsorted(m, min(gd[j], rd[j])))
            assert abs(c[lo] - dus[j]) < 1e-4, (j, gd, rd)
    gm.close()

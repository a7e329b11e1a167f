"""GPU parity of the recent-window KV variant (kv_window W > 0): the last W
positions of every attention layer are read at fp16 from a ring, older ones
from their int8 / 3-bit codes (page 3, Qwen3.8-27B 實測, section "RTX 4090
24GB").  Checked against the oracle with the same window: teacher-forced steps
on the toy stack across the window boundary (outputs, appended codes and the
appended fp16 ring entry), free-running greedy decoding, and the full-size
attention layer (d = 256, 6 q heads per kv head, W = 2048) on a synthetic
4096-position cache and ring."""
import sys

import numpy as np
import pytest

import oracle
import synth
from synth import state as SS
from synth import workloads as W
from tests.helpers import rel_l2
from tests.test_gpu_parity import TOL, TOL_STEP, _tie_checked

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


def _gpu_model(A, shape, seed, graph=True):
    from synth.gpu_load import load_recipe
    m = A.Model(shape, graph=graph)
    load_recipe(m, shape, seed)
    return m


def _import(gm, om, shape):
    for l, t in enumerate(shape.pattern):
        if t == "G":
            gm.import_gdn(l, om.get_gdn_state(l).astype(np.float32))
        else:
            gm.import_kv(l, *om.get_kv(l, om.pos))
            gm.import_win(l, *om.get_win(l))
    gm.set_pos(om.pos)


def _f16(b):
    return np.asarray(b, np.uint16).view(np.float16).astype(np.float64)


def _ring_entry_close(g, o):
    """fp16 entries of one appended key or rotated value: the fp32 values they
    are rounded from differ by the perturbation that fp16 re-rounding of the
    projection's input produces (about 1e-4 of the vector's scale, the bound
    the code checks use), plus one fp16 step of the entry itself"""
    gv, ov = _f16(g), _f16(o)
    step = np.maximum(np.abs(ov), 2.0 ** -14) * 2.0 ** -10
    return bool(np.all(np.abs(gv - ov) <= 1e-3 * np.max(np.abs(ov)) + step))


def test_window_toy_teacher_forced(aw4):
    """TOY stack with W = 16: 44 teacher-forced steps from the oracle's state,
    positions 0..43, so the window first holds every position and then slides."""
    import torch
    shape = W.with_(W.TOY, kv_window=16)
    _say("case: toy stack, window 16, teacher-forced 44 steps")
    om = oracle.from_recipe(shape, 2)
    gm = _gpu_model(aw4, shape, 2)
    toks = synth.tokens(44, shape.vocab, 2)
    logits = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    clean, tied = [], []
    for i in range(44):
        t = int(toks[i])
        _import(gm, om, shape)
        pos = om.pos
        xo, lo, ao = om.decode_token(t)
        ag = gm.decode_step(t, logits)
        xg, lg = gm.read_hidden(), logits.cpu().numpy()
        err = max(rel_l2(xg, xo), rel_l2(lg, lo))
        flips = 0
        for l, lt in enumerate(shape.pattern):
            if lt != "A":
                continue
            gk, ok = gm.export_kv(l, pos + 1), om.get_kv(l, pos + 1)
            gw, ow = gm.export_win(l), om.get_win(l)
            slot = pos % shape.kv_window
            # the other slots came from the oracle, unchanged
            others = [s for s in range(shape.kv_window) if s != slot]
            assert np.array_equal(gw[0][others], ow[0][others]) and np.array_equal(gw[1][others], ow[1][others])
            if flips:
                continue
            assert _ring_entry_close(gw[0][slot], ow[0][slot]), (i, l)
            assert _ring_entry_close(gw[1][slot], ow[1][slot]), (i, l)
            kv, vv = om.last_kv(l)
            flips += _tie_checked(gk[0][pos].reshape(-1, 32), ok[0][pos].reshape(-1, 32), gk[1][pos].ravel(),
                                  ok[1][pos].ravel(), kv.reshape(-1, 32), 127)
            flips += _tie_checked(gk[2][pos].reshape(-1, 32), ok[2][pos].reshape(-1, 32), gk[3][pos].ravel(),
                                  ok[3][pos].ravel(), vv.reshape(-1, 32), 3)
        if ag != ao:
            top = np.sort(lo)[-2:]
            assert top[1] - top[0] < 1e-3 * np.std(lo), (i, ag, ao)
        (tied if flips else clean).append(err)
    _say(f"clean steps {len(clean)} worst {max(clean):.2e}; steps with tie flips {len(tied)}")
    assert len(clean) >= 22
    assert max(clean) < TOL_STEP
    assert not tied or max(tied) < 0.1
    gm.close()


def test_window_toy_free_running(aw4):
    """TOY stack with W = 24: a 64-token prompt (token by token: chunked prefill
    does not read the window) then 96 greedy steps on each side."""
    shape = W.with_(W.TOY, kv_window=24)
    _say("case: toy stack, window 24, 64 prompt + 96 greedy")
    prompt = synth.tokens(64, shape.vocab, 3)
    gm = _gpu_model(aw4, shape, 3)
    gm.prefill(prompt[:-1])
    g = gm.decode_greedy(int(prompt[-1]), 96)
    xg = gm.read_hidden()
    om = oracle.from_recipe(shape, 3)
    for t in prompt[:-1]:
        om.decode_token(int(t))
    tok, ref = int(prompt[-1]), []
    for _ in range(96):
        x, lo, tok = om.decode_token(tok)
        ref.append(tok)
    _say(f"final hidden rel-L2 {rel_l2(xg, x):.2e}")
    assert list(g) == ref
    assert rel_l2(xg, x) < TOL
    gm.close()


def test_window_differs_from_codes_only(aw4):
    """The same toy run with and without the window gives different hidden
    states on the GPU (the ring is read), and the window run equals the
    oracle's window run, not its codes-only run."""
    _say("case: toy stack, window 8 vs none")
    prompt = synth.tokens(40, W.TOY.vocab, 4)
    xs = {}
    for win in (0, 8):
        shape = W.with_(W.TOY, kv_window=win)
        gm = _gpu_model(aw4, shape, 4)
        gm.prefill(prompt)
        xs[win] = gm.read_hidden()
        gm.close()
        om = oracle.from_recipe(shape, 4)
        for t in prompt:
            xo, _, _ = om.decode_token(int(t))
        xs[("o", win)] = xo
    assert rel_l2(xs[8], xs[("o", 8)]) < TOL
    assert rel_l2(xs[8], xs[("o", 0)]) > 10 * rel_l2(xs[8], xs[("o", 8)])


@pytest.mark.parametrize("npos", [1000, 4096])
def test_window_attention_layer_full_size(aw4, npos):
    """Full-size gated-attention layer with W = 2048 on a synthetic cache and
    ring: 4 teacher-forced steps through the layer (window longer than the
    cache at 1000 positions; both parts read at 4096)."""
    import torch
    shape = W.with_(W.ATTN_LAYER, max_ctx=max(npos, 2048) + 64, kv_window=2048)
    _say("case: full-size attention layer, window 2048, cache", npos)
    om = oracle.from_recipe(shape, 6)
    gm = _gpu_model(aw4, shape, 6)
    SS.fill(om, shape, npos, 6)
    SS.fill(gm, shape, npos, 6)
    xin = synth.normal(4, shape.hidden, 1.0, 6, W.STREAM_HIDDEN)
    xd = torch.empty(shape.hidden, dtype=torch.float32, device="cuda")
    worst = 0.0
    for t in range(4):
        _import(gm, om, shape)
        xd.copy_(torch.from_numpy(xin[t]))
        torch.cuda.synchronize()
        gm.decode_hidden(xd, xd)
        gm.sync()
        xo = om.forward_layers(xin[t].astype(np.float64))
        worst = max(worst, rel_l2(xd.cpu().numpy() - xin[t], xo - xin[t]))
    _say(f"worst layer-delta rel-L2 {worst:.2e}")
    assert worst < TOL
    gm.close()


def test_window_rejects_paths_without_it(aw4):
    shape = W.with_(W.TOY, kv_window=8)
    _say("case: window rejections")
    gm = _gpu_model(aw4, shape, 1)
    gm.prefill(synth.tokens(4, shape.vocab, 1))
    with pytest.raises(aw4.AW4Error):
        gm.verify_k([1, 2])
    with pytest.raises(aw4.AW4Error):
        gm.set_prefill_chunk(16)
    with pytest.raises(aw4.AW4Error):
        gm.decode_batch([1])
    gm.close()


def test_window_graph_equals_eager(aw4):
    """The decode step with a window, replayed from its captured graph, gives
    the tokens and hidden state of the same steps launched kernel by kernel."""
    shape = W.with_(W.TOY, kv_window=12)
    _say("case: toy stack, window 12, graph vs eager, 24 prompt + 24 greedy")
    prompt = synth.tokens(24, shape.vocab, 5)
    out = []
    for graph in (True, False):
        gm = _gpu_model(aw4, shape, 5, graph=graph)
        gm.prefill(prompt[:-1])
        toks = gm.decode_greedy(int(prompt[-1]), 24)
        out.append((list(toks), gm.read_hidden()))
        gm.close()
    assert out[0][0] == out[1][0]
    assert np.array_equal(out[0][1], out[1][1])

"""GPU checks of the boundary's states: a model computes only once every
tensor of its config holds values; a weight blob (attention_w4_amd.blob, the
oracle codec's logical tensors) loads through aw4_load_weights and decodes as
the oracle does; a bad blob changes nothing; an injected HIP failure comes back
as AW4_E_HIP and the model recovers after a reset; a recent window with one kv
head at a context whose split count meets the combine's limit decodes; moving
the position back with a window needs the ring re-imported."""
import sys

import numpy as np
import pytest

import oracle
import synth
from synth import workloads as W
from tests.helpers import logical_weights, oracle_from_logical, rel_l2

pytestmark = pytest.mark.gpu

E_HIP, E_FORMAT, E_STATE = -4, -5, -8


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


def _items(shape, seed):
    out = []
    for (layer, kind), v in logical_weights(shape, seed).items():
        if kind == W.T_RHT_SIGNS:
            v = np.asarray(v, np.float32)
        out.append((layer, kind, v))
    return out


def _code(e):
    return getattr(e, "code", None)


def _greedy_vs_oracle(gm, om, prompt, n):
    gm.prefill(prompt[:-1])
    got = list(gm.decode_greedy(int(prompt[-1]), n))
    xg = gm.read_hidden()
    for t in prompt[:-1]:
        om.decode_token(int(t))
    tok, ref, x = int(prompt[-1]), [], None
    for _ in range(n):
        x, _, tok = om.decode_token(tok)
        ref.append(tok)
    return got, ref, rel_l2(xg, x)


def test_blob_loads_and_decodes_like_the_oracle(aw4):
    from attention_w4_amd import blob
    shape, seed = W.TOY, 9
    _say("case: toy stack loaded from a blob, 8-token prompt + 16 greedy steps")
    items = _items(shape, seed)
    b = blob.write_blob(aw4.Config.from_shape(shape), items)
    assert aw4.check_blob(shape, b) == 0
    gm = aw4.Model(shape)
    # nothing loaded: every call that runs the model refuses
    for call in (lambda: gm.decode_step(1), lambda: gm.prefill([1, 2]), lambda: gm.decode_greedy(1, 2)):
        with pytest.raises(aw4.AW4Error) as ei:
            call()
        assert _code(ei.value) == E_STATE
    # all but one vector: still refused
    gm.load_weights(blob.write_blob(aw4.Config.from_shape(shape), items[:-1]))
    with pytest.raises(aw4.AW4Error) as ei:
        gm.decode_step(1)
    assert _code(ei.value) == E_STATE
    gm.load_weights(b)
    om = oracle_from_logical(shape, logical_weights(shape, seed))
    prompt = synth.tokens(8, shape.vocab, seed)
    got, ref, err = _greedy_vs_oracle(gm, om, prompt, 16)
    _say(f"tokens equal {got == ref}, hidden rel-L2 {err:.2e}")
    assert got == ref and err < 1e-2
    # a bad blob (its last tensor's first value non-finite) is refused whole and
    # the loaded weights stay: the same continuation again from a reset
    bad = bytearray(b)
    bad[-4:] = np.float32(np.nan).tobytes()
    with pytest.raises(aw4.AW4Error) as ei:
        gm.load_weights(bytes(bad))
    assert _code(ei.value) == E_FORMAT
    gm.reset()
    om2 = oracle_from_logical(shape, logical_weights(shape, seed))
    got2, ref2, err2 = _greedy_vs_oracle(gm, om2, prompt, 16)
    assert got2 == ref2 == ref and err2 < 1e-2
    gm.close()


@pytest.mark.parametrize("n", [1, 3, 40])
def test_injected_hip_failure_returns_e_hip(aw4, n):
    """the n-th checked HIP call of a decode step reports failure: the step
    returns AW4_E_HIP; after a reset the model decodes as the oracle does"""
    from synth.gpu_load import load_recipe
    shape, seed = W.TOY, 4
    _say("case: injected HIP failure at checked call", n)
    gm = aw4.Model(shape, graph=(n != 40))
    load_recipe(gm, shape, seed)
    aw4.test_fail_hip_call(n)
    try:
        with pytest.raises(aw4.AW4Error) as ei:
            for _ in range(64):   # the countdown ends inside one of these steps
                gm.decode_step(3)
        assert _code(ei.value) == E_HIP
    finally:
        aw4.test_fail_hip_call(0)
    gm.sync()
    gm.reset()
    om = oracle.from_recipe(shape, seed)
    got, ref, err = _greedy_vs_oracle(gm, om, synth.tokens(6, shape.vocab, seed), 8)
    assert got == ref and err < 1e-2
    gm.close()


def test_window_with_one_kv_head_at_4k_decodes(aw4):
    """TOY (one kv head) with max_ctx 4096 and a window of 16: the main sweep
    takes 255 split slots so that with the window's slot the combine's 256 are
    not exceeded; greedy decoding matches the oracle.  Moving the position back
    then refuses to decode until the rings are imported again."""
    from synth.gpu_load import load_recipe
    shape, seed = W.with_(W.TOY, kv_window=16, max_ctx=4096), 6
    _say("case: toy, one kv head, max_ctx 4096, window 16")
    gm = aw4.Model(shape)
    load_recipe(gm, shape, seed)
    om = oracle.from_recipe(shape, seed)
    got, ref, err = _greedy_vs_oracle(gm, om, synth.tokens(24, shape.vocab, seed), 24)
    _say(f"tokens equal {got == ref}, hidden rel-L2 {err:.2e}")
    assert got == ref and err < 1e-2
    p = gm.pos
    gm.set_pos(p - 4)
    with pytest.raises(aw4.AW4Error) as ei:
        gm.decode_step(1)
    assert _code(ei.value) == E_STATE
    alayers = [l for l, t in enumerate(shape.pattern) if t == "A"]
    for l in alayers:
        gm.import_win(l, *gm.export_win(l))
    gm.decode_step(1)   # accepted once every ring was imported
    gm.close()

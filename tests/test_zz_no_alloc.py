"""GPU check of aw4_decode_step_static, the decode step whose split partials
and head partials live in the library's static device scratch: its outputs
equal aw4_decode_step's (the same kernels; only where the partials sit
differs) on consecutive calls, the second at a smaller context than the
first, so the scratch still holds the first call's partials in slots the
second does not use; a step that needs more static scratch than the library
holds is refused with AW4_E_INVAL."""
import sys

import numpy as np
import pytest

import synth
from synth import workloads as W

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


def test_static_step_equals_decode_step(aw4):
    import torch
    from synth.gpu_load import load_recipe
    shape = W.with_(W.TOY, max_ctx=1024)
    ga, gb = aw4.Model(shape), aw4.Model(shape)
    for g in (ga, gb):
        load_recipe(g, shape, 3)
    la = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    lb = torch.empty_like(la)
    for n_prompt in (601, 9):   # 38 of 64 attention splits in use, then 1
        _say("case: static-scratch decode step after a prompt of", n_prompt)
        prompt = synth.tokens(n_prompt, shape.vocab, 3 + n_prompt)
        for g in (ga, gb):
            g.reset()
            g.prefill(prompt[:-1])
        ta, tb = int(prompt[-1]), int(prompt[-1])
        for step in range(4):
            ta = ga.decode_step(ta, la)
            tb = gb.decode_step_static(tb, lb)
            torch.cuda.synchronize()
            assert ta == tb, (n_prompt, step)
            assert torch.equal(la, lb), (n_prompt, step)
            assert np.array_equal(ga.read_hidden(), gb.read_hidden()), (n_prompt, step)
        assert ga.pos == gb.pos == n_prompt - 1 + 4
    ga.close()
    gb.close()


def test_static_step_refuses_a_step_beyond_its_scratch(aw4):
    """64 query heads over 8 kv heads at d = 256 with a 4096-position window:
    32 + 64 split slots per row, 6.3 MB of partials, above the 4 MiB held"""
    shape = W.with_(W.TOY, pattern="A", attn_q_heads=64, attn_kv_heads=8, attn_head_dim=256,
                    max_ctx=8192, kv_window=4096)
    _say("case: static-scratch step refused (6.3 MB of partials)")
    g = aw4.Model(shape)
    with pytest.raises(aw4.AW4Error) as ei:
        g.decode_step_static(1)
    assert ei.value.code == -1
    g.close()

"""GPU parity of batch decode (aw4_decode_batch, aw4_select_sequence): B
sequences, each with its own states, caches and position, take one greedy step
together.  The definition is B independent decode steps, so each sequence is
checked against its own oracle model run token by token: greedy tokens must be
identical, and a sequence selected afterwards continues from the state the
batch left.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from synth import state as SS
from synth import workloads as W
from tests.helpers import rel_l2

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


def test_batch_toy_matches_oracle_sequences(aw4):
    from synth.gpu_load import load_recipe
    _say("case: toy stack, 4 sequences (prompts of 20, 33, 47, 8 tokens), batch steps of 4, 3 and 1")
    shape = W.with_(W.TOY, max_batch=4)
    lens = [20, 33, 47, 8]
    prompts = [synth.tokens(n, shape.vocab, 30 + b) for b, n in enumerate(lens)]
    gm = aw4.Model(shape)
    load_recipe(gm, shape, 3)
    first = []
    for b, p in enumerate(prompts):
        gm.select_sequence(b)
        gm.prefill(p[:-1])
        first.append(int(p[-1]))
    gm.select_sequence(0)
    oms = []
    for b, p in enumerate(prompts):
        om = oracle.from_recipe(shape, 3)
        for t in p[:-1]:
            om.decode_token(int(t))
        oms.append(om)
    cur = list(first)
    got = [[] for _ in range(4)]
    schedule = [4] * 8 + [3] * 4 + [1] * 2 + [4] * 2
    for B in schedule:
        out = gm.decode_batch(cur[:B])
        for b in range(B):
            got[b].append(out[b])
            cur[b] = out[b]
    ref = [[] for _ in range(4)]
    for b in range(4):
        tok = first[b]
        for _ in range(len(got[b])):
            _, _, tok = oms[b].decode_token(tok)
            ref[b].append(tok)
    for b in range(4):
        assert got[b] == ref[b], b
    # a selected sequence continues where the batch left it
    gm.select_sequence(2)
    assert gm.pos == lens[2] - 1 + len(got[2])
    x = gm.decode_step(cur[2])
    _, _, t = oms[2].decode_token(cur[2])
    assert x == t
    gm.close()


def test_batch_full_size_from_synthetic_states(aw4):
    """The 27B-shape stack: two sequences from different 1024-position
    synthetic states, four batch steps, against the oracle per sequence."""
    import torch
    from synth.gpu_load import load_recipe
    _say("case: full 27B-shape stack, 2 sequences from 1024-position states, 4 batch steps")
    shape = W.with_(W.FULL_27B, max_ctx=1100, max_batch=2)
    gm = aw4.Model(shape)
    load_recipe(gm, shape, 0)
    seeds = [0, 1]
    for b, sd in enumerate(seeds):
        gm.select_sequence(b)
        SS.fill(gm, shape, 1024, sd)
    first = [int(synth.tokens(1, shape.vocab, sd, i0=1024)[0]) for sd in seeds]
    cur, got = list(first), [[], []]
    for _ in range(4):
        out = gm.decode_batch(cur)
        for b in range(2):
            got[b].append(out[b])
        cur = out
    gm.close()
    del gm
    torch.cuda.empty_cache()
    om = oracle.from_recipe(W.with_(shape, max_batch=1), 0)
    for b, sd in enumerate(seeds):
        SS.fill(om, shape, 1024, sd)
        ref, tok = [], first[b]
        for _ in range(4):
            _, _, tok = om.decode_token(tok)
            ref.append(tok)
        _say(f"sequence {b}: gpu {got[b]} oracle {ref}")
        assert got[b] == ref


def test_batch_graph_equals_eager(aw4):
    """The batch step replayed from its captured graph (one per batch size,
    captured on first use) gives the tokens of the same step launched kernel
    by kernel, over a schedule that returns to a batch size already captured."""
    from synth.gpu_load import load_recipe
    _say("case: toy stack, 3 sequences, batch steps of 3, 2, 3 with and without graphs")
    shape = W.with_(W.TOY, max_batch=3)
    lens = [12, 25, 9]
    prompts = [synth.tokens(n, shape.vocab, 50 + b) for b, n in enumerate(lens)]
    res = []
    for graph in (True, False):
        gm = aw4.Model(shape)
        load_recipe(gm, shape, 7)
        gm.set_graph(graph)
        for b, p in enumerate(prompts):
            gm.select_sequence(b)
            gm.prefill(p[:-1])
        gm.select_sequence(0)
        cur = [int(p[-1]) for p in prompts]
        seqs = []
        for B in [3] * 5 + [2] * 3 + [3] * 4:
            out = gm.decode_batch(cur[:B])
            seqs.append(tuple(out))
            cur[:B] = out
        # the states the batch left, read through a single-sequence step
        gm.select_sequence(1)
        seqs.append(gm.decode_step(cur[1]))
        res.append((seqs, gm.read_hidden()))
        gm.close()
    assert res[0][0] == res[1][0]
    assert np.array_equal(res[0][1], res[1][1])

"""Writes tests/golden/full_27b_greedy_8k.json: the oracle's 256 greedy tokens
of the full 27B-shape stack (64 layers, vocab 248320, seeded recipe weights,
no draft head) from the seeded synthetic 8192-position state; per step its four
largest logits (ids and values), and the residual (hidden state) after steps
32, 64, 96, 128, 192 and 256 as base64 of little-endian float32.

Calls only oracle/ (and the seeded input generators in synth/); the GPU test
test_gpu_full.py::test_full_27b_greedy_256 compares the library against this
file, since the oracle needs minutes for 256 full-size steps.

    python tests/golden/make_full_greedy.py [steps]
"""
import base64
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402
from synth import state as SS  # noqa: E402
from synth import workloads as W  # noqa: E402

CTX, SEED = 8192, 0
SNAPS = (32, 64, 96, 128, 192, 256)
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "full_27b_greedy_8k.json")


def shape_for(steps):
    return W.with_(W.FULL_27B, max_ctx=CTX + steps + 8, draft_vocab=0)


def main(steps=256):
    shape = shape_for(steps)
    t0 = time.time()
    om = oracle.from_recipe(shape, SEED)
    SS.fill(om, shape, CTX, SEED)
    print(f"oracle built in {time.time() - t0:.0f} s", flush=True)
    first = int(synth.tokens(1, shape.vocab, SEED, i0=CTX)[0])
    tok, toks, margins, top, snaps = first, [], [], [], {}
    t0 = time.time()
    for i in range(steps):
        x, lo, tok = om.decode_token(tok)
        ids = np.argsort(-lo, kind="stable")[:4]
        top.append([[int(j) for j in ids], [float(lo[j]) for j in ids]])
        margins.append(float(lo[ids[0]] - lo[ids[1]]))
        toks.append(int(tok))
        if i + 1 in SNAPS:
            snaps[str(i + 1)] = base64.b64encode(np.asarray(x, "<f4").tobytes()).decode()
        if i % 16 == 15:
            print(f"step {i + 1}: {time.time() - t0:.0f} s", flush=True)
    out = {"what": "oracle greedy tokens of the full 27B-shape stack (seeded recipe weights, seed 0, no draft "
                   "head) from the seeded synthetic 8192-position state",
           "script": "tests/golden/make_full_greedy.py", "ctx": CTX, "seed": SEED, "first": first,
           "steps": steps, "tokens": toks, "min_top2_margin": min(margins),
           "margins_below_1e-3": int(sum(m < 1e-3 for m in margins)),
           "top4": top, "hidden_after": snaps,
           "final_hidden": [float(np.float32(v)) for v in x]}
    with open(OUT, "w") as f:
        json.dump(out, f)
    print("wrote", OUT, "min margin", min(margins))


if __name__ == "__main__":
    main(int(sys.argv[1]) if len(sys.argv) > 1 else 256)

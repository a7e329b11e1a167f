"""Consistency of the stored oracle runs under tests/golden/ (no GPU, no
oracle run): each file names the script that wrote it, and its fields agree
with each other, so a truncated or hand-edited file fails here rather than as
a puzzling GPU mismatch."""
import base64
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_full_greedy_golden_is_consistent():
    g = json.load(open(os.path.join(GOLDEN, "full_27b_greedy_8k.json")))
    assert g["script"] == "tests/golden/make_full_greedy.py"
    assert os.path.exists(os.path.join(GOLDEN, "make_full_greedy.py"))
    n = g["steps"]
    assert n == 256 and len(g["tokens"]) == n and len(g["top4"]) == n
    margins = []
    for tok, (ids, vals) in zip(g["tokens"], g["top4"]):
        assert ids[0] == tok and len(set(ids)) == 4
        assert all(vals[j] >= vals[j + 1] for j in range(3))
        assert all(0 <= i < 248320 for i in ids)
        margins.append(vals[0] - vals[1])
    assert abs(min(margins) - g["min_top2_margin"]) < 1e-12
    assert g["margins_below_1e-3"] == sum(m < 1e-3 for m in margins)
    assert sorted(int(k) for k in g["hidden_after"]) == [32, 64, 96, 128, 192, 256]
    for v in g["hidden_after"].values():
        x = np.frombuffer(base64.b64decode(v), "<f4")
        assert x.shape == (5120,) and np.all(np.isfinite(x))
    last = np.frombuffer(base64.b64decode(g["hidden_after"]["256"]), "<f4")
    assert np.array_equal(last, np.asarray(g["final_hidden"], np.float32))

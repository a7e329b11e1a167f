"""Host-side checks of the benchmark's accounting (no GPU): the algorithmic
bytes a decode step is priced at, against the model's own tensor list and the
library's cache layout, and the refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

import bench
from synth import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _matrix_bytes(spec):
    """stored bytes of a matrix: its codes (4 or 8 bits) and one fp16 scale per 32 columns"""
    code_bits = {W.W4: 4, W.I8: 8}[spec.fmt]
    return spec.rows * spec.cols * code_bits // 8 + spec.rows * (spec.cols // 32) * 2


@pytest.mark.parametrize("name", ["FULL_27B", "TOY"])
def test_step_bytes_match_the_tensor_list(name):
    """The weights part of step_bytes is every target-model matrix the loaders
    set (draft head excluded: a decode step does not read it), each once."""
    s = getattr(W, name)
    n = s.n_layers
    mats = [t for t in W.tensor_specs(s) if t.fmt in (W.W4, W.I8) and t.layer != n]
    weights = sum(_matrix_bytes(t) for t in mats)
    ng, na = s.pattern.count("G"), s.pattern.count("A")
    rest = (s.vocab * 4 + ng * s.gdn_v_heads * s.gdn_head_dim ** 2 * 8
            + na * bench.kv_bytes_per_pos(s) * 101)
    assert bench.step_bytes(s, 100) == weights + rest


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_cache_bytes_match_the_library_layout(fmt):
    """kv_bytes_per_pos prices exactly what the library stores per position:
    the arena grows by that much per attention layer (and per draft-head
    cache, which has the same row format) for every added position.  Formats
    1 and 2 serve no draft head, so their shape drops it."""
    import attention_w4_amd as A
    s = W.with_(W.FULL_27B, kv_format=fmt, draft_vocab=W.FULL_27B.draft_vocab if fmt == 0 else 0)
    caches = s.pattern.count("A") + (1 if s.draft_vocab > 0 else 0)
    a = A.workspace_bytes(W.with_(s, max_ctx=8192))
    b = A.workspace_bytes(W.with_(s, max_ctx=8192 + 1024))
    assert b - a == caches * bench.kv_bytes_per_pos(s) * 1024


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]

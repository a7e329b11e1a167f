"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/aw4.h declares, and validates configs and arenas
on the host without enqueuing anything."""
import ctypes
import os
import re

import pytest

import attention_w4_amd as A
from synth import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "aw4.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(aw4_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = A.lib()
    names = declared_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(L, n), n
    # the binding wraps all of them
    assert set(names) <= set(A.exported_symbols())


def _cfg(shape, **kw):
    c = A.Config.from_shape(shape)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("shape", [W.TOY, W.FULL_27B, W.GDN_LAYER, W.ATTN_LAYER,
                                   W.with_(W.TOY, kv_window=16), W.with_(W.FULL_27B, kv_window=2048, draft_vocab=0)])
def test_valid_configs(shape):
    assert A.lib().aw4_validate_config(ctypes.byref(_cfg(shape))) == 0


def test_window_adds_its_ring_to_the_workspace():
    """kv_window W adds two fp16 rings of W x nkv x dh per attention layer
    (and W / 64 split slots of partials)"""
    base = A.workspace_bytes(W.TOY)
    win = A.workspace_bytes(W.with_(W.TOY, kv_window=64))
    ring = 2 * 64 * W.TOY.attn_kv_heads * W.TOY.attn_head_dim * 2
    assert ring <= win - base <= ring + 4096 + 4 * W.TOY.attn_q_heads * (W.TOY.attn_head_dim + 2) * 4


@pytest.mark.parametrize("kw", [
    dict(hidden=100), dict(ffn=0), dict(group=16), dict(n_layers=3), dict(layer_pattern=b"GX"),
    dict(gdn_head_dim=96), dict(attn_head_dim=128), dict(attn_q_heads=6, attn_kv_heads=4),
    dict(gdn_v_heads=6, gdn_qk_heads=4), dict(max_verify=5), dict(max_verify=0), dict(rms_eps=0.0),
    dict(vocab=-1), dict(max_ctx=0), dict(attn_q_heads=3, attn_kv_heads=1),
    dict(kv_window=-1), dict(kv_window=2000), dict(kv_window=16, max_batch=2),
    dict(kv_window=16, draft_vocab=64),
])
def test_invalid_configs(kw):
    c = _cfg(W.TOY, **kw)
    assert A.lib().aw4_validate_config(ctypes.byref(c)) == -1
    out = ctypes.c_uint64()
    assert A.lib().aw4_workspace_bytes(ctypes.byref(c), ctypes.byref(out)) == -1


def test_workspace_bytes_full_model():
    n = A.workspace_bytes(W.FULL_27B)
    # W4 layer weights 12.843 GB + int8 head 1.351 GB (4.5 and 8.5 bits per weight),
    # GDN state 48 * 2 MiB... plus the KV cache for max_ctx positions; the draft
    # head's W4 block and fuse (424.7 M weights), its cache and its id maps; the
    # prefill chunk buffers for 1024 tokens
    s = W.FULL_27B
    H, F, C = s.hidden, s.ffn, 1024
    kv_pos = s.attn_kv_heads * (s.attn_head_dim * (1 + 3 / 8) + 4 * s.attn_head_dim / 32)
    kv = 17 * kv_pos * s.max_ctx
    weights = 14_194_278_400 + 424_673_280 * 9 // 16 + 4 * (s.draft_vocab + s.vocab)
    state = 48 * s.gdn_v_heads * s.gdn_head_dim ** 2 * 4
    nvd, nqd = s.gdn_v_heads * s.gdn_head_dim, s.attn_q_heads * s.attn_head_dim
    prefill = C * (4 * H + 2 * 2 * H + 2 * F + 4 * (2 * nqd + 2 * 1024) + 4 * nvd + 8 * s.gdn_qk_heads * s.gdn_head_dim
                   + 8 * s.gdn_v_heads + 4 * s.attn_q_heads * (s.attn_head_dim + 2))
    need = weights + state + kv + prefill
    assert need < n < need * 1.02


def test_create_rejects_bad_arena_without_touching_device():
    c = _cfg(W.TOY)
    h = ctypes.c_void_p()
    assert A.lib().aw4_create(ctypes.byref(c), None, 1 << 30, None, ctypes.byref(h)) == -2
    assert A.lib().aw4_create(ctypes.byref(c), ctypes.c_void_p(256), 16, None, ctypes.byref(h)) == -2
    assert A.lib().aw4_create(ctypes.byref(c), ctypes.c_void_p(257), 1 << 40, None, ctypes.byref(h)) == -2
    assert not h.value


def test_null_model_calls_are_rejected():
    L = A.lib()
    assert L.aw4_reset(None) == -1
    assert L.aw4_decode_step(None, 0, None, None) == -1
    assert L.aw4_decode_greedy(None, 0, 1, None) == -1
    assert L.aw4_prefill(None, None, 0, None) == -1
    assert L.aw4_status_string(-6) == b"context full"
    assert L.aw4_last_error(None) == b"null model"
    L.aw4_destroy(None)

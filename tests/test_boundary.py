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
                                   W.with_(W.TOY, kv_window=16), W.with_(W.FULL_27B, kv_window=2048, draft_vocab=0),
                                   W.with_(W.TOY, kv_format=1), W.with_(W.FULL_27B, kv_format=2, draft_vocab=0)])
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
    dict(kv_format=3), dict(kv_format=-1), dict(kv_format=1, kv_window=16), dict(kv_format=2, max_batch=2),
    dict(kv_format=1, draft_vocab=64),
])
def test_invalid_configs(kw):
    c = _cfg(W.TOY, **kw)
    assert A.lib().aw4_validate_config(ctypes.byref(c)) == -1
    out = ctypes.c_uint64()
    assert A.lib().aw4_workspace_bytes(ctypes.byref(c), ctypes.byref(out)) == -1


def test_cache_formats_size_the_workspace():
    """per attention layer, kv head and position: format 0 and 2 hold a key row
    of d bytes and a value record of 3 d / 8 bytes, format 1 (q4_0) d / 2 bytes
    each; the scales are the same"""
    s = W.with_(W.ATTN_LAYER, draft_vocab=0)
    n = s.attn_kv_heads * s.max_ctx
    d = s.attn_head_dim
    b0, b1, b2 = (A.workspace_bytes(W.with_(s, kv_format=f)) for f in (0, 1, 2))
    assert b2 == b0
    assert abs((b0 - b1) - n * (d + 3 * d // 8 - d // 2 - d // 2)) <= 4096


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


# ------------------------------------------------------------- weight blob (pure host)
def _blob_items(shape, seed=3):
    """(layer, kind, value) of every tensor: the oracle codec's logical codes
    and scales, fp32 vectors, signs as fp32, the draft map as int32"""
    import numpy as np
    from tests.helpers import logical_weights
    items = []
    for (layer, kind), v in logical_weights(shape, seed).items():
        if kind == W.T_RHT_SIGNS:
            v = np.asarray(v, np.float32)
        items.append((layer, kind, v))
    return items


@pytest.fixture(scope="module")
def tiny_blob():
    from attention_w4_amd import blob
    from tests.helpers import TINY_MTP
    return TINY_MTP, blob.write_blob(A.Config.from_shape(TINY_MTP), _blob_items(TINY_MTP))


def _records(b):
    """offsets of every tensor record of a well-formed blob"""
    import struct
    from attention_w4_amd import blob
    off = len(blob.header(A.Config.from_shape(W.TOY), 0))
    (count,) = struct.unpack_from("<I", b, off - 4)
    out = []
    for _ in range(count):
        layer, kind, rows, cols, nb = struct.unpack_from("<iiqqQ", b, off)
        out.append((off, layer, kind, rows, cols, nb))
        off += 32 + nb
    assert off == len(b)
    return out


def test_blob_checks_clean(tiny_blob):
    shape, b = tiny_blob
    assert A.check_blob(shape, b) == 0
    # any subset of the tensors is a valid blob
    from attention_w4_amd import blob
    assert A.check_blob(shape, blob.write_blob(A.Config.from_shape(shape), [])) == 0
    assert A.check_blob(shape, blob.write_blob(A.Config.from_shape(shape), _blob_items(shape)[:3])) == 0


def _set(b, off, fmt, val):
    import struct
    bb = bytearray(b)
    struct.pack_into(fmt, bb, off, val)
    return bytes(bb)


def test_blob_rejects_every_malformation(tiny_blob):
    import struct
    shape, b = tiny_blob
    F = -5
    recs = _records(b)
    mat = next(r for r in recs if r[2] == W.T_MIX_IN)
    vec = next(r for r in recs if r[2] == W.T_NORM_MIX)
    sig = next(r for r in recs if r[2] == W.T_RHT_SIGNS)
    mp = next(r for r in recs if r[2] == W.T_DRAFT_MAP)
    head = next(r for r in recs if r[2] == W.T_LM_HEAD)
    cases = {
        "magic": b"AW4X" + b[4:],
        "version": _set(b, 4, "<I", 3),
        "echo hidden": _set(b, 8, "<i", shape.hidden + 64),
        "echo draft_vocab": _set(b, 8 + 4 * 11, "<i", shape.draft_vocab + 1),
        "echo pattern": b[:56] + b"GAAG" + b[60:],
        "count too high": _set(b, 184, "<I", len(recs) + 1),
        "count too low": _set(b, 184, "<I", len(recs) - 1),
        "truncated header": b[:100],
        "truncated payload": b[:-1],
        "trailing byte": b + b"\0",
        "rows": _set(b, mat[0] + 8, "<q", mat[3] + 1),
        "cols": _set(b, vec[0] + 16, "<q", vec[4] + 32),
        "payload bytes": _set(b, vec[0] + 24, "<Q", vec[5] + 4),
        "kind not in config": _set(b, vec[0] + 4, "<i", W.T_DRAFT_NORM_EMB),   # a draft-head kind at a target layer
        "layer out of range": _set(b, mat[0], "<i", len(shape.pattern) + 1),
        "w4 code -8": _set(b, mat[0] + 32 + 5, "<B", 0x80),
        "int8 code -128": _set(b, head[0] + 32 + 7, "<b", -128),
        "scale nan": _set(b, mat[0] + 32 + mat[3] * mat[4] // 2 + 2, "<H", 0x7E00),
        "scale negative": _set(b, mat[0] + 32 + mat[3] * mat[4] // 2, "<H", 0xB800),
        "vector inf": _set(b, vec[0] + 32 + 8, "<f", float("inf")),
        "sign not +-1": _set(b, sig[0] + 32, "<f", 0.5),
        "map id repeated": _set(b, mp[0] + 32 + 4, "<i", struct.unpack_from("<i", b, mp[0] + 32)[0]),
        "map id out of range": _set(b, mp[0] + 32, "<i", shape.vocab),
        "duplicate tensor": (b[:184] + struct.pack("<I", len(recs) + 1) + b[188:] +
                             b[vec[0]:vec[0] + 32 + vec[5]]),
    }
    assert vec[1] < len(shape.pattern)
    for name, bad in cases.items():
        assert A.check_blob(shape, bad) == F, name
    assert A.check_blob(W.with_(shape, ffn=shape.ffn + 64), b) == F


def test_blob_check_rejects_bad_arguments(tiny_blob):
    shape, b = tiny_blob
    L = A.lib()
    c = A.Config.from_shape(shape)
    assert L.aw4_check_blob(ctypes.byref(c), None, 16) == -1
    bad = A.Config.from_shape(shape)
    bad.group = 16
    assert A.check_blob(bad, b) == -1


def test_blob_writer_round_trips_the_records(tiny_blob):
    """the records the writer emits carry each tensor's shape and its bytes in
    order: codes then scales, vectors as fp32"""
    import numpy as np
    shape, b = tiny_blob
    items = _blob_items(shape)
    recs = _records(b)
    assert [(r[1], r[2]) for r in recs] == [(l, k) for l, k, _ in items]
    for (off, layer, kind, rows, cols, nb), (_, _, v) in zip(recs, items):
        payload = b[off + 32: off + 32 + nb]
        if kind in (0, 1, 2, 3, 4, 5, 12):
            codes, scales = v
            assert rows == scales.shape[0] and cols == scales.shape[1] * 32
            assert payload == np.ascontiguousarray(codes).tobytes() + np.ascontiguousarray(scales, np.uint16).tobytes()
        elif kind == W.T_DRAFT_MAP:
            assert payload == np.asarray(v, np.int32).tobytes()
        else:
            assert payload == np.asarray(v, np.float32).tobytes()


def test_fault_hook_is_exported():
    L = A.lib()
    assert L.aw4_test_fail_hip_call(0) == 0

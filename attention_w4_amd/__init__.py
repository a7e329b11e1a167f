"""Python binding of libaw4.so (batch-1 hybrid W4 decode on MI355X / gfx950).

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind the C ABI declared in include/aw4.h.  PyTorch supplies the
device arena and the stream.  There is no fallback: if the library is missing
or the device is not gfx950, the calls raise.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libaw4.so")

AW4_OK = 0
STATUS = {0: "ok", -1: "AW4_E_INVAL", -2: "AW4_E_ARENA", -3: "AW4_E_NODEVICE", -4: "AW4_E_HIP",
          -5: "AW4_E_FORMAT", -6: "AW4_E_CTX_FULL", -7: "AW4_E_TOKEN", -8: "AW4_E_STATE"}

T_MIX_IN, T_MIX_OUT, T_FFN_GATE, T_FFN_UP, T_FFN_DOWN, T_LM_HEAD = 0, 1, 2, 3, 4, 5
T_NORM_MIX, T_NORM_FFN, T_NORM_GATED, T_A_BIAS, T_NORM_FINAL, T_RHT_SIGNS = 6, 7, 8, 9, 10, 11
T_DRAFT_FUSE, T_DRAFT_NORM_EMB, T_DRAFT_NORM_HID, T_DRAFT_NORM_OUT, T_DRAFT_MAP = 12, 13, 14, 15, 16
PHASE_FFN_GATE_UP, PHASE_FFN_DOWN, PHASE_MIX_IN, PHASE_HEAD, PHASE_DRAFT_HEAD = 0, 1, 2, 3, 4
PHASE_PREFILL_GATE_UP = 5

_i32, _i64, _u64, _f32, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float, ctypes.c_void_p


class Config(ctypes.Structure):
    _fields_ = [("hidden", _i32), ("ffn", _i32), ("vocab", _i32), ("n_layers", _i32),
                ("gdn_qk_heads", _i32), ("gdn_v_heads", _i32), ("gdn_head_dim", _i32),
                ("attn_q_heads", _i32), ("attn_kv_heads", _i32), ("attn_head_dim", _i32),
                ("group", _i32), ("max_ctx", _i32), ("max_verify", _i32), ("rms_eps", _f32),
                ("layer_pattern", ctypes.c_char * 128), ("draft_vocab", _i32), ("max_batch", _i32),
                ("kv_window", _i32), ("kv_format", _i32)]

    @classmethod
    def from_shape(cls, s):
        c = cls()
        for f in ("hidden", "ffn", "vocab", "gdn_qk_heads", "gdn_v_heads", "gdn_head_dim",
                  "attn_q_heads", "attn_kv_heads", "attn_head_dim", "group", "max_ctx", "max_verify"):
            setattr(c, f, int(getattr(s, f)))
        c.n_layers = len(s.pattern)
        c.rms_eps = float(s.rms_eps)
        c.layer_pattern = s.pattern.encode()
        c.draft_vocab = int(getattr(s, "draft_vocab", 0))
        c.max_batch = int(getattr(s, "max_batch", 1))
        c.kv_window = int(getattr(s, "kv_window", 0))
        c.kv_format = int(getattr(s, "kv_format", 0))
        return c


class AW4Error(RuntimeError):
    def __init__(self, code, what, detail=""):
        super().__init__(f"{what}: {STATUS.get(code, code)} {detail}".strip())
        self.code = code


_lib = None

_SIGS = {
    "aw4_validate_config": [ctypes.c_void_p],
    "aw4_workspace_bytes": [ctypes.c_void_p, ctypes.POINTER(_u64)],
    "aw4_create": [ctypes.c_void_p, _vp, _u64, _vp, ctypes.POINTER(_vp)],
    "aw4_tensor_shape": [_vp, _i32, _i32, ctypes.POINTER(_i64), ctypes.POINTER(_i64)],
    "aw4_quantize_tensor": [_vp, _i32, _i32, _i64, _i64, _vp],
    "aw4_load_tensor": [_vp, _i32, _i32, _vp, _vp],
    "aw4_export_tensor": [_vp, _i32, _i32, _vp, _vp],
    "aw4_set_vector": [_vp, _i32, _i32, _vp, _i32],
    "aw4_set_draft_map": [_vp, _vp, _i32],
    "aw4_load_weights": [_vp, _vp, _u64],
    "aw4_reset": [_vp],
    "aw4_prefill": [_vp, _vp, _i32, _vp],
    "aw4_set_prefill_chunk": [_vp, _i32],
    "aw4_decode_step": [_vp, _i32, _vp, _vp],
    "aw4_decode_greedy": [_vp, _i32, _i32, _vp],
    "aw4_decode_hidden": [_vp, _vp, _vp],
    "aw4_verify_k": [_vp, _vp, _i32, _vp, _vp, _f32, _vp, _vp],
    "aw4_draft": [_vp, _i32, _i32, _f32, _vp, _vp, _vp, _vp],
    "aw4_read_hidden": [_vp, _vp],
    "aw4_set_graph": [_vp, _i32],
    "aw4_get_pos": [_vp, ctypes.POINTER(_i32)],
    "aw4_set_pos": [_vp, _i32],
    "aw4_get_draft_pos": [_vp, ctypes.POINTER(_i32)],
    "aw4_set_draft_pos": [_vp, _i32],
    "aw4_select_sequence": [_vp, _i32],
    "aw4_decode_batch": [_vp, _vp, _i32, _vp],
    "aw4_time_phase": [_vp, _i32, _i32, ctypes.POINTER(_f32), ctypes.POINTER(_u64)],
    "aw4_export_state_gdn": [_vp, _i32, _vp],
    "aw4_import_state_gdn": [_vp, _i32, _vp],
    "aw4_export_state_kv": [_vp, _i32, _i32, _vp, _vp, _vp, _vp],
    "aw4_import_state_kv": [_vp, _i32, _i32, _vp, _vp, _vp, _vp],
    "aw4_export_state_win": [_vp, _i32, _vp, _vp],
    "aw4_import_state_win": [_vp, _i32, _vp, _vp],
    "aw4_check_blob": [ctypes.c_void_p, _vp, _u64],
    "aw4_test_fail_hip_call": [_i32],
    "aw4_decode_step_static": [_vp, _i32, _vp, _vp],
    "aw4_time_stream_read": [_vp, _u64, _vp, _vp, _i32, ctypes.POINTER(_f32)],
}


def lib():
    """Load libaw4.so; raises if it is missing (no fallback path exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build()")
        # torch first: its bundled HIP runtime then serves this library too (same
        # soname), so device pointers and streams come from one runtime instance
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.aw4_destroy.argtypes = [_vp]
        L.aw4_destroy.restype = None
        L.aw4_status_string.argtypes = [ctypes.c_int]
        L.aw4_status_string.restype = ctypes.c_char_p
        L.aw4_last_error.argtypes = [_vp]
        L.aw4_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def exported_symbols():
    return ["aw4_destroy", "aw4_status_string", "aw4_last_error"] + list(_SIGS)


def workspace_bytes(shape):
    c = Config.from_shape(shape)
    out = _u64()
    rc = lib().aw4_workspace_bytes(ctypes.byref(c), ctypes.byref(out))
    if rc != AW4_OK:
        raise AW4Error(rc, "aw4_workspace_bytes")
    return out.value


def _ptr(a):
    """host numpy array -> void*"""
    return a.ctypes.data_as(ctypes.c_void_p)


def _blob_ptr(blob):
    """(pointer, length) of a bytes-like blob, without a copy"""
    import numpy as np
    a = np.frombuffer(blob, np.uint8) if len(blob) else np.zeros(1, np.uint8)
    return _ptr(a), len(blob), a


def check_blob(shape_or_cfg, blob):
    """aw4_check_blob: 0 for a blob that loads into this config, else the status"""
    c = shape_or_cfg if isinstance(shape_or_cfg, Config) else Config.from_shape(shape_or_cfg)
    p, n, _keep = _blob_ptr(blob)
    return lib().aw4_check_blob(ctypes.byref(c), p, n)


def time_stream_read(buf, sink, stream, reps):
    """aw4_time_stream_read over a device tensor buf (its bytes); sink: a
    device tensor of at least 8 KB; stream: a torch stream.  -> average us"""
    us = _f32()
    nbytes = buf.numel() * buf.element_size() // 16 * 16
    rc = lib().aw4_time_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), stream.cuda_stream, int(reps),
                                    ctypes.byref(us))
    if rc != AW4_OK:
        raise AW4Error(rc, "aw4_time_stream_read")
    return us.value


def test_fail_hip_call(n):
    """arm (n >= 1) or disarm (n <= 0) the library's HIP failure injection"""
    lib().aw4_test_fail_hip_call(int(n))


class Model:
    """A model bound to a torch-allocated device arena and a dedicated stream."""

    def __init__(self, shape, device="cuda:0", graph=True):
        import torch
        self.shape = shape
        self.cfg = Config.from_shape(shape)
        self.device = torch.device(device)
        nbytes = workspace_bytes(shape)
        with torch.cuda.device(self.device):
            self.arena = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            # a non-default stream (default priority) so the step can be captured as a graph
            self.stream = torch.cuda.Stream(device=self.device)
            h = _vp()
            rc = lib().aw4_create(ctypes.byref(self.cfg), self.arena.data_ptr(), nbytes,
                                  self.stream.cuda_stream, ctypes.byref(h))
        if rc != AW4_OK:
            raise AW4Error(rc, "aw4_create")
        self.h = h
        self.set_graph(graph)

    def close(self):
        if getattr(self, "h", None):
            lib().aw4_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _rc(self, rc, what):
        if rc != AW4_OK:
            raise AW4Error(rc, what, lib().aw4_last_error(self.h).decode())

    def sync(self):
        self.stream.synchronize()

    # ---------------------------------------------------------------- weights
    def tensor_shape(self, layer, kind):
        r, c = _i64(), _i64()
        self._rc(lib().aw4_tensor_shape(self.h, layer, kind, ctypes.byref(r), ctypes.byref(c)), "tensor_shape")
        return r.value, c.value

    def quantize_tensor(self, layer, kind, row0, src):
        """src: fp32 device tensor [nrows, cols] (contiguous) on this model's device."""
        assert src.is_cuda and src.is_contiguous() and src.dtype.itemsize == 4
        self._rc(lib().aw4_quantize_tensor(self.h, layer, kind, row0, src.shape[0], src.data_ptr()),
                 "quantize_tensor")

    def load_tensor(self, layer, kind, codes, scales):
        import numpy as np
        codes = np.ascontiguousarray(codes)
        scales = np.ascontiguousarray(scales, np.uint16)
        self._rc(lib().aw4_load_tensor(self.h, layer, kind, _ptr(codes), _ptr(scales)), "load_tensor")

    def export_tensor(self, layer, kind):
        import numpy as np
        rows, cols = self.tensor_shape(layer, kind)
        if kind == T_LM_HEAD:
            codes = np.zeros((rows, cols), np.int8)
        else:
            codes = np.zeros((rows, cols // 2), np.uint8)
        scales = np.zeros((rows, cols // 32), np.uint16)
        self._rc(lib().aw4_export_tensor(self.h, layer, kind, _ptr(codes), _ptr(scales)), "export_tensor")
        return codes, scales

    def set_vector(self, layer, kind, vals):
        import numpy as np
        v = np.ascontiguousarray(vals, np.float32)
        self._rc(lib().aw4_set_vector(self.h, layer, kind, _ptr(v), len(v)), "set_vector")

    def set_draft_map(self, ids):
        import numpy as np
        v = np.ascontiguousarray(ids, np.int32)
        self._rc(lib().aw4_set_draft_map(self.h, _ptr(v), len(v)), "set_draft_map")

    def load_weights(self, blob):
        """blob: bytes-like in the aw4_load_weights format (attention_w4_amd.blob)"""
        p, n, _keep = _blob_ptr(blob)
        self._rc(lib().aw4_load_weights(self.h, p, n), "load_weights")

    # ---------------------------------------------------------------- decode
    def reset(self):
        self._rc(lib().aw4_reset(self.h), "reset")

    def set_graph(self, enable):
        self._rc(lib().aw4_set_graph(self.h, 1 if enable else 0), "set_graph")

    @property
    def pos(self):
        p = _i32()
        self._rc(lib().aw4_get_pos(self.h, ctypes.byref(p)), "get_pos")
        return p.value

    def set_pos(self, p):
        self._rc(lib().aw4_set_pos(self.h, p), "set_pos")

    def prefill(self, tokens, logits=None):
        import numpy as np
        t = np.ascontiguousarray(tokens, np.int32)
        self._rc(lib().aw4_prefill(self.h, _ptr(t), len(t), logits.data_ptr() if logits is not None else None),
                 "prefill")

    def set_prefill_chunk(self, n):
        """prompt tokens per prefill chunk (0: token by token)"""
        self._rc(lib().aw4_set_prefill_chunk(self.h, int(n)), "set_prefill_chunk")

    def decode_step(self, token, logits=None, want_argmax=True):
        am = _i32()
        self._rc(lib().aw4_decode_step(self.h, int(token), logits.data_ptr() if logits is not None else None,
                                       ctypes.byref(am) if want_argmax else None), "decode_step")
        return am.value if want_argmax else None

    def decode_step_static(self, token, logits=None, want_argmax=True):
        """aw4_decode_step_static: the decode step with its partials in the
        library's static device scratch"""
        am = _i32()
        self._rc(lib().aw4_decode_step_static(self.h, int(token), logits.data_ptr() if logits is not None else None,
                                              ctypes.byref(am) if want_argmax else None), "decode_step_static")
        return am.value if want_argmax else None

    def decode_greedy(self, first_token, n):
        import numpy as np
        out = np.zeros(max(n, 1), np.int32)
        self._rc(lib().aw4_decode_greedy(self.h, int(first_token), n, _ptr(out)), "decode_greedy")
        return out[:n]

    def verify_k(self, tokens, q=None, u=None, temperature=0.0):
        """tokens: [t0, d1..dk]; q: device fp32 tensor [k, V] (sampling); u: k+1 uniforms.
        Returns the emitted tokens (accepted drafts + the drawn token)."""
        import numpy as np
        t = np.ascontiguousarray(tokens, np.int32)
        k = len(t) - 1
        uu = np.ascontiguousarray(u, np.float32) if u is not None else None
        out = np.zeros(4, np.int32)
        n = _i32()
        self._rc(lib().aw4_verify_k(self.h, _ptr(t), k, q.data_ptr() if q is not None else None,
                                    _ptr(uu) if uu is not None else None, float(temperature), _ptr(out),
                                    ctypes.byref(n)), "verify_k")
        return [int(v) for v in out[:n.value]]

    def draft(self, t0, k, temperature=0.0, u=None, q=None, scores=None):
        """k drafts from the draft head after the last committed position, t0 the
        token run next.  q: device fp32 tensor [k, vocab] receiving the draft
        probabilities (temperature > 0); scores: device fp32 tensor [k,
        draft_vocab] receiving the mapped scores; u: k uniforms."""
        import numpy as np
        uu = np.ascontiguousarray(u, np.float32) if u is not None else None
        out = np.zeros(4, np.int32)
        self._rc(lib().aw4_draft(self.h, int(t0), int(k), float(temperature), _ptr(uu) if uu is not None else None,
                                 q.data_ptr() if q is not None else None,
                                 scores.data_ptr() if scores is not None else None, _ptr(out)), "draft")
        return [int(v) for v in out[:k]]

    def select_sequence(self, s):
        self._rc(lib().aw4_select_sequence(self.h, int(s)), "select_sequence")

    def decode_batch(self, tokens):
        """one greedy step for sequences 0 .. len(tokens) - 1; returns their argmax tokens"""
        import numpy as np
        t = np.ascontiguousarray(tokens, np.int32)
        out = np.zeros(4, np.int32)
        self._rc(lib().aw4_decode_batch(self.h, _ptr(t), len(t), _ptr(out)), "decode_batch")
        return [int(v) for v in out[:len(t)]]

    @property
    def dpos(self):
        p = _i32()
        self._rc(lib().aw4_get_draft_pos(self.h, ctypes.byref(p)), "get_draft_pos")
        return p.value

    def set_dpos(self, p):
        self._rc(lib().aw4_set_draft_pos(self.h, p), "set_draft_pos")

    def decode_hidden(self, x_in, x_out):
        self._rc(lib().aw4_decode_hidden(self.h, x_in.data_ptr(), x_out.data_ptr()), "decode_hidden")

    def read_hidden(self):
        import numpy as np
        x = np.zeros(self.shape.hidden, np.float32)
        self._rc(lib().aw4_read_hidden(self.h, _ptr(x)), "read_hidden")
        return x

    def time_phase(self, phase, reps):
        """(average microseconds per launch, algorithmic bytes per launch)"""
        us, b = _f32(), _u64()
        self._rc(lib().aw4_time_phase(self.h, phase, reps, ctypes.byref(us), ctypes.byref(b)), "time_phase")
        return us.value, b.value

    # ---------------------------------------------------------------- state
    def export_gdn(self, layer):
        import numpy as np
        s = self.shape
        S = np.zeros((s.gdn_v_heads, s.gdn_head_dim, s.gdn_head_dim), np.float32)
        self._rc(lib().aw4_export_state_gdn(self.h, layer, _ptr(S)), "export_state_gdn")
        return S

    def import_gdn(self, layer, S):
        import numpy as np
        S = np.ascontiguousarray(S, np.float32)
        self._rc(lib().aw4_import_state_gdn(self.h, layer, _ptr(S)), "import_state_gdn")

    def export_kv(self, layer, npos):
        import numpy as np
        s = self.shape
        d, nkv = s.attn_head_dim, s.attn_kv_heads
        kc = np.zeros((npos, nkv, d), np.int8)
        vc = np.zeros((npos, nkv, d), np.int8)
        ks = np.zeros((npos, nkv, d // 32), np.uint16)
        vs = np.zeros((npos, nkv, d // 32), np.uint16)
        self._rc(lib().aw4_export_state_kv(self.h, layer, npos, _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs)),
                 "export_state_kv")
        return kc, ks, vc, vs

    def import_kv(self, layer, kc, ks, vc, vs):
        import numpy as np
        arrs = [np.ascontiguousarray(kc, np.int8), np.ascontiguousarray(ks, np.uint16),
                np.ascontiguousarray(vc, np.int8), np.ascontiguousarray(vs, np.uint16)]
        self._rc(lib().aw4_import_state_kv(self.h, layer, arrs[0].shape[0], *[_ptr(a) for a in arrs]),
                 "import_state_kv")

    def export_win(self, layer):
        """recent-window ring (fp16 bits of keys, rotated values) [W][nkv][dh]"""
        import numpy as np
        s = self.shape
        kw = np.zeros((s.kv_window, s.attn_kv_heads, s.attn_head_dim), np.uint16)
        vw = np.zeros_like(kw)
        self._rc(lib().aw4_export_state_win(self.h, layer, _ptr(kw), _ptr(vw)), "export_state_win")
        return kw, vw

    def import_win(self, layer, kw, vw):
        import numpy as np
        kw, vw = (np.ascontiguousarray(a, np.uint16) for a in (kw, vw))
        self._rc(lib().aw4_import_state_win(self.h, layer, _ptr(kw), _ptr(vw)), "import_state_win")

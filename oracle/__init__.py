"""CPU oracle of the hybrid W4 decode step (TEST INFRASTRUCTURE ONLY).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
this package.  It shares no code with the HIP library: the C model in
aw4_oracle.c is compiled with gcc and driven through ctypes here; brute.py is
an independent numpy implementation for tiny shapes; accept.py holds the
speculative-decoding acceptance rule.

Precision and formats are described in aw4_oracle.c.  Each function is
pinned by CPU tests (tests/test_oracle_*.py) against values the pages and the
mathematics fix, not against itself.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(_HERE, "liboracle.so")

_vp, _i32, _i64, _f32, _f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double


def build():
    src = os.path.join(_HERE, "aw4_oracle.c")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                           "-o", SO + ".tmp", src, "-lm"])
    os.replace(SO + ".tmp", SO)
    global _lib
    _lib = None


class Cfg(ctypes.Structure):
    _fields_ = [("hidden", _i32), ("ffn", _i32), ("vocab", _i32), ("n_layers", _i32),
                ("gdn_qk_heads", _i32), ("gdn_v_heads", _i32), ("gdn_head_dim", _i32),
                ("attn_q_heads", _i32), ("attn_kv_heads", _i32), ("attn_head_dim", _i32),
                ("group", _i32), ("max_ctx", _i32), ("rms_eps", _f64), ("pattern", ctypes.c_char * 128),
                ("draft_vocab", _i32), ("kv_window", _i32), ("kv_format", _i32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(SO):
            raise RuntimeError(f"{SO} missing: run __graft_entry__.build()")
        L = ctypes.CDLL(SO)
        sig = {
            "or_f32_to_f16": ([_f32], ctypes.c_uint16),
            "or_f16_to_f64": ([ctypes.c_uint16], _f64),
            "or_quant_group": ([_vp, ctypes.c_int, ctypes.c_int, _vp, _vp], None),
            "or_quant_w4_rows": ([_vp, _i64, _i64, _vp, _vp], None),
            "or_quant_i8_rows": ([_vp, _i64, _i64, _vp, _vp], None),
            "or_rht_forward": ([_vp, _vp, ctypes.c_int, _vp], None),
            "or_rht_inverse": ([_vp, _vp, ctypes.c_int, _vp], None),
            "or_create": ([ctypes.POINTER(Cfg)], _vp),
            "or_destroy": ([_vp], None),
            "or_load_w4": ([_vp, ctypes.c_int, ctypes.c_int, _vp, _vp], ctypes.c_int),
            "or_quant_w4_into": ([_vp, ctypes.c_int, ctypes.c_int, _i64, _i64, _vp], ctypes.c_int),
            "or_quant_lm_into": ([_vp, _i64, _i64, _vp], ctypes.c_int),
            "or_load_i8": ([_vp, _vp, _vp], ctypes.c_int),
            "or_load_vec": ([_vp, ctypes.c_int, ctypes.c_int, _vp, ctypes.c_int], ctypes.c_int),
            "or_load_signs": ([_vp, _vp, ctypes.c_int], ctypes.c_int),
            "or_gdn_head_step": ([_vp, _vp, _vp, _vp, _f64, _f64, ctypes.c_int, ctypes.c_int, _vp], None),
            "or_attend_head": ([_vp, _vp, _vp, _vp, _vp, _i64, _i64, ctypes.c_int, _vp, _vp, _vp, _i64, _i64, _vp],
                               None),
            "or_kv_encode": ([_vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _vp], None),
            "or_kv_encode_fmt": ([_vp, _vp, _vp, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _vp], None),
            "or_attend_head_fmt": ([_vp, _vp, _vp, _vp, _vp, _i64, _i64, ctypes.c_int, _vp, _vp, _vp, _i64, _i64,
                                    ctypes.c_int, _vp], None),
            "or_lm_level": ([ctypes.c_int], _f64),
            "or_quant_group_lm": ([_vp, ctypes.c_int, _vp, _vp], None),
            "or_forward_layers": ([_vp, _vp, _vp], ctypes.c_int),
            "or_embed": ([_vp, _i32, _vp], ctypes.c_int),
            "or_head": ([_vp, _vp, _vp, _vp], ctypes.c_int),
            "or_decode_token": ([_vp, _i32, _vp, _vp, _vp], ctypes.c_int),
            "or_get_pos": ([_vp], _i32),
            "or_set_pos": ([_vp, _i32], ctypes.c_int),
            "or_get_last_kv": ([_vp, ctypes.c_int, _vp, _vp], ctypes.c_int),
            "or_set_state_win": ([_vp, ctypes.c_int, _vp, _vp], ctypes.c_int),
            "or_get_state_win": ([_vp, ctypes.c_int, _vp, _vp], ctypes.c_int),
            "or_set_state_gdn": ([_vp, ctypes.c_int, _vp], ctypes.c_int),
            "or_get_state_gdn": ([_vp, ctypes.c_int, _vp], ctypes.c_int),
            "or_set_state_gdn64": ([_vp, ctypes.c_int, _vp], ctypes.c_int),
            "or_set_state_kv": ([_vp, ctypes.c_int, _i32, _vp, _vp, _vp, _vp], ctypes.c_int),
            "or_set_draft_map": ([_vp, _vp, _i32], ctypes.c_int),
            "or_get_draft_map": ([_vp, _vp], ctypes.c_int),
            "or_draft_step": ([_vp, _i32, _vp, _i32, _vp, _vp], ctypes.c_int),
            "or_get_dpos": ([_vp], _i32),
            "or_set_dpos": ([_vp, _i32], ctypes.c_int),
            "or_get_state_kv": ([_vp, ctypes.c_int, _i32, _vp, _vp, _vp, _vp], ctypes.c_int),
        }
        for name, (a, r) in sig.items():
            f = getattr(L, name)
            f.argtypes = a
            f.restype = r
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


# ------------------------------------------------------------------ codec helpers
def f32_to_f16_bits(x):
    return np.array([lib().or_f32_to_f16(float(v)) for v in np.asarray(x, np.float32).ravel()],
                    dtype=np.uint16).reshape(np.shape(x))


def f16_bits_to_f64(h):
    return np.array([lib().or_f16_to_f64(int(v)) for v in np.asarray(h, np.uint16).ravel()],
                    dtype=np.float64).reshape(np.shape(h))


def quant_group(x, qmax):
    x = np.ascontiguousarray(x, dtype=np.float32)
    s = np.zeros(1, np.uint16)
    c = np.zeros(len(x), np.int8)
    lib().or_quant_group(_p(x), len(x), qmax, _p(s), _p(c))
    return int(s[0]), c


def quant_w4(w):
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 32), np.uint16)
    lib().or_quant_w4_rows(_p(w), rows, cols, _p(codes), _p(scales))
    return codes, scales


def quant_i8(w):
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    codes = np.zeros((rows, cols), np.int8)
    scales = np.zeros((rows, cols // 32), np.uint16)
    lib().or_quant_i8_rows(_p(w), rows, cols, _p(codes), _p(scales))
    return codes, scales


def rht_forward(v, signs):
    v = np.ascontiguousarray(v, np.float64)
    s = np.ascontiguousarray(signs, np.int8)
    out = np.zeros_like(v)
    lib().or_rht_forward(_p(v), _p(s), len(v), _p(out))
    return out


def rht_inverse(v, signs):
    v = np.ascontiguousarray(v, np.float64)
    s = np.ascontiguousarray(signs, np.int8)
    out = np.zeros_like(v)
    lib().or_rht_inverse(_p(v), _p(s), len(v), _p(out))
    return out


def gdn_head_step(S, k, v, q, alpha, beta):
    """One head: returns (new S, o).  S is [dv][dk]."""
    S = np.array(S, np.float64, order="C")
    dv, dk = S.shape
    k, v, q = (np.ascontiguousarray(a, np.float64) for a in (k, v, q))
    o = np.zeros(dv)
    lib().or_gdn_head_step(_p(S), _p(k), _p(v), _p(q), alpha, beta, dv, dk, _p(o))
    return S, o


def lm_levels():
    """the Lloyd-Max codebook of the value-cache format 2, ascending (fp16 values)"""
    return np.array([lib().or_lm_level(c) for c in range(8)])


def quant_group_lm(x):
    """the codebook codec of one group: (scale bits, level indices 0..7)"""
    x = np.ascontiguousarray(x, dtype=np.float32)
    s = np.zeros(1, np.uint16)
    c = np.zeros(len(x), np.int8)
    lib().or_quant_group_lm(_p(x), len(x), _p(s), _p(c))
    return int(s[0]), c


def attend_head(q, kc, ks, vc, vs, signs, kw=None, vw=None, fmt=0):
    """q [d]; kc/vc int8 [npos][d]; ks/vs fp16 bits [npos][d/32].  With a window
    ring kw/vw (fp16 bits [W][d], position t at slot t % W), the last W
    positions are read from it instead of the codes.  fmt: the cache format
    (0: V codes -3..3 rotated; 1: 4-bit K and V, V not rotated; 2: V codebook
    indices 0..7 rotated)."""
    q = np.ascontiguousarray(q, np.float64)
    kc, vc = np.ascontiguousarray(kc, np.int8), np.ascontiguousarray(vc, np.int8)
    ks, vs = np.ascontiguousarray(ks, np.uint16), np.ascontiguousarray(vs, np.uint16)
    sg = np.ascontiguousarray(signs, np.int8)
    npos, d = kc.shape
    out = np.zeros(d)
    if kw is None:
        lib().or_attend_head_fmt(_p(q), _p(kc), _p(ks), _p(vc), _p(vs), npos, d, d, _p(sg), None, None, 0, 0,
                                 fmt, _p(out))
    else:
        kw, vw = np.ascontiguousarray(kw, np.uint16), np.ascontiguousarray(vw, np.uint16)
        lib().or_attend_head_fmt(_p(q), _p(kc), _p(ks), _p(vc), _p(vs), npos, d, d, _p(sg), _p(kw), _p(vw),
                                 kw.shape[0], d, fmt, _p(out))
    return out


def kv_encode(k, v, signs, fmt=0):
    d = len(k)
    k, v = np.ascontiguousarray(k, np.float64), np.ascontiguousarray(v, np.float64)
    sg = np.ascontiguousarray(signs, np.int8)
    kc, vc = np.zeros(d, np.int8), np.zeros(d, np.int8)
    ks, vs = np.zeros(d // 32, np.uint16), np.zeros(d // 32, np.uint16)
    lib().or_kv_encode_fmt(_p(k), _p(v), _p(sg), d, fmt, _p(kc), _p(ks), _p(vc), _p(vs))
    return kc, ks, vc, vs


# ------------------------------------------------------------------ model
T_MIX_IN, T_MIX_OUT, T_FFN_GATE, T_FFN_UP, T_FFN_DOWN, T_LM_HEAD = 0, 1, 2, 3, 4, 5
T_NORM_MIX, T_NORM_FFN, T_NORM_GATED, T_A_BIAS, T_NORM_FINAL, T_RHT_SIGNS = 6, 7, 8, 9, 10, 11
T_DRAFT_FUSE, T_DRAFT_NORM_EMB, T_DRAFT_NORM_HID, T_DRAFT_NORM_OUT = 12, 13, 14, 15


class Model:
    """The oracle model.  shape: any object with the fields of synth.workloads.Shape."""

    def __init__(self, shape):
        self.shape = shape
        c = Cfg()
        for f in ("hidden", "ffn", "vocab", "gdn_qk_heads", "gdn_v_heads", "gdn_head_dim",
                  "attn_q_heads", "attn_kv_heads", "attn_head_dim", "group", "max_ctx"):
            setattr(c, f, int(getattr(shape, f)))
        c.n_layers = len(shape.pattern)
        c.rms_eps = float(shape.rms_eps)
        c.pattern = shape.pattern.encode()
        c.draft_vocab = int(getattr(shape, "draft_vocab", 0))
        c.kv_window = int(getattr(shape, "kv_window", 0))
        c.kv_format = int(getattr(shape, "kv_format", 0))
        self._cfg = c
        self.h = lib().or_create(ctypes.byref(c))
        if not self.h:
            raise MemoryError("oracle allocation failed")

    def __del__(self):
        if getattr(self, "h", None) and _lib is not None:
            _lib.or_destroy(self.h)
            self.h = None

    def _rc(self, rc, what):
        if rc != 0:
            raise ValueError(f"oracle {what} failed ({rc})")

    # -- weights
    def load_w4(self, layer, kind, codes, scales):
        codes = np.ascontiguousarray(codes, np.uint8)
        scales = np.ascontiguousarray(scales, np.uint16)
        self._rc(lib().or_load_w4(self.h, layer, kind, _p(codes), _p(scales)), "load_w4")

    def quant_w4_into(self, layer, kind, row0, w):
        w = np.ascontiguousarray(w, np.float32)
        self._rc(lib().or_quant_w4_into(self.h, layer, kind, row0, w.shape[0], _p(w)), "quant_w4_into")

    def quant_lm_into(self, row0, w):
        w = np.ascontiguousarray(w, np.float32)
        self._rc(lib().or_quant_lm_into(self.h, row0, w.shape[0], _p(w)), "quant_lm_into")

    def load_i8(self, codes, scales):
        codes = np.ascontiguousarray(codes, np.int8)
        scales = np.ascontiguousarray(scales, np.uint16)
        self._rc(lib().or_load_i8(self.h, _p(codes), _p(scales)), "load_i8")

    def load_vec(self, layer, kind, v):
        v = np.ascontiguousarray(v, np.float32)
        self._rc(lib().or_load_vec(self.h, layer, kind, _p(v), len(v)), "load_vec")

    def load_signs(self, s):
        s = np.ascontiguousarray(s, np.int8)
        self._rc(lib().or_load_signs(self.h, _p(s), len(s)), "load_signs")

    # -- steps
    @property
    def pos(self):
        return lib().or_get_pos(self.h)

    def set_pos(self, p):
        self._rc(lib().or_set_pos(self.h, p), "set_pos")

    def forward_layers(self, x, trace=False):
        x = np.array(x, np.float64)
        tr = np.zeros((len(self.shape.pattern), self.shape.hidden)) if trace else None
        self._rc(lib().or_forward_layers(self.h, _p(x), _p(tr) if trace else None), "forward_layers")
        return (x, tr) if trace else x

    def embed(self, token):
        x = np.zeros(self.shape.hidden)
        self._rc(lib().or_embed(self.h, int(token), _p(x)), "embed")
        return x

    def head(self, x):
        x = np.ascontiguousarray(x, np.float64)
        logits = np.zeros(self.shape.vocab)
        am = np.zeros(1, np.int32)
        self._rc(lib().or_head(self.h, _p(x), _p(logits), _p(am)), "head")
        return logits, int(am[0])

    def decode_token(self, token):
        """-> (final residual, logits, argmax)"""
        x = np.zeros(self.shape.hidden)
        logits = np.zeros(self.shape.vocab)
        am = np.zeros(1, np.int32)
        self._rc(lib().or_decode_token(self.h, int(token), _p(x), _p(logits), _p(am)), "decode_token")
        return x, logits, int(am[0])

    # -- draft head (layer index n_layers holds its weights)
    def set_draft_map(self, ids):
        ids = np.ascontiguousarray(ids, np.int32)
        self._rc(lib().or_set_draft_map(self.h, _p(ids), len(ids)), "set_draft_map")

    def draft_map(self):
        ids = np.zeros(self.shape.draft_vocab, np.int32)
        self._rc(lib().or_get_draft_map(self.h, _p(ids)), "draft_map")
        return ids

    @property
    def dpos(self):
        return lib().or_get_dpos(self.h)

    def set_dpos(self, p):
        self._rc(lib().or_set_dpos(self.h, p), "set_dpos")

    def draft_step(self, token, h, slot=0):
        """-> (output hidden [H], mapped logits [draft_vocab]); writes draft cache
        entry dpos + slot, leaves dpos unchanged"""
        h = np.ascontiguousarray(h, np.float64)
        x = np.zeros(self.shape.hidden)
        z = np.zeros(self.shape.draft_vocab)
        self._rc(lib().or_draft_step(self.h, int(token), _p(h), int(slot), _p(x), _p(z)), "draft_step")
        return x, z

    # -- state
    def set_gdn_state(self, layer, S):
        S = np.ascontiguousarray(S, np.float32)
        self._rc(lib().or_set_state_gdn(self.h, layer, _p(S)), "set_gdn_state")

    def get_gdn_state(self, layer):
        s = self.shape
        S = np.zeros((s.gdn_v_heads, s.gdn_head_dim, s.gdn_head_dim))
        self._rc(lib().or_get_state_gdn(self.h, layer, _p(S)), "get_gdn_state")
        return S

    def set_kv(self, layer, kc, ks, vc, vs):
        npos = kc.shape[0]
        arrs = [np.ascontiguousarray(a) for a in (kc, ks, vc, vs)]
        self._rc(lib().or_set_state_kv(self.h, layer, npos, *[_p(a) for a in arrs]), "set_kv")

    def last_kv(self, layer):
        """fp32 keys and rotated values [nkv][dh] the last append quantised"""
        s = self.shape
        k = np.zeros((s.attn_kv_heads, s.attn_head_dim), np.float32)
        v = np.zeros_like(k)
        self._rc(lib().or_get_last_kv(self.h, layer, _p(k), _p(v)), "last_kv")
        return k, v

    def get_win(self, layer):
        """fp16 window ring (keys, rotated values) [W][nkv][dh] as uint16 bits"""
        s = self.shape
        kw = np.zeros((s.kv_window, s.attn_kv_heads, s.attn_head_dim), np.uint16)
        vw = np.zeros_like(kw)
        self._rc(lib().or_get_state_win(self.h, layer, _p(kw), _p(vw)), "get_win")
        return kw, vw

    def set_win(self, layer, kw, vw):
        kw, vw = (np.ascontiguousarray(a, np.uint16) for a in (kw, vw))
        self._rc(lib().or_set_state_win(self.h, layer, _p(kw), _p(vw)), "set_win")

    def snapshot(self):
        """recurrent states, caches (and fp16 windows) and position"""
        st = {"pos": self.pos}
        win = getattr(self.shape, "kv_window", 0)
        for l, t in enumerate(self.shape.pattern):
            st[l] = self.get_gdn_state(l) if t == "G" else self.get_kv(l, self.pos)
            if t == "A" and win > 0:
                st[("win", l)] = self.get_win(l)
        return st

    def restore(self, st):
        for l, t in enumerate(self.shape.pattern):
            if t == "G":
                S = np.ascontiguousarray(st[l], np.float64)
                self._rc(lib().or_set_state_gdn64(self.h, l, _p(S)), "restore")
            else:
                self.set_kv(l, *st[l])
                if ("win", l) in st:
                    self.set_win(l, *st[("win", l)])
        self.set_pos(st["pos"])

    def get_kv(self, layer, npos):
        s = self.shape
        d, nkv = s.attn_head_dim, s.attn_kv_heads
        kc = np.zeros((npos, nkv, d), np.int8)
        vc = np.zeros((npos, nkv, d), np.int8)
        ks = np.zeros((npos, nkv, d // 32), np.uint16)
        vs = np.zeros((npos, nkv, d // 32), np.uint16)
        self._rc(lib().or_get_state_kv(self.h, layer, npos, _p(kc), _p(ks), _p(vc), _p(vs)), "get_kv")
        return kc, ks, vc, vs


def from_recipe(shape, seed, norm_jitter=0.0, chunk_rows=None):
    """Build an oracle model whose fp32 weights come from the seeded recipe
    (synth.workloads.tensor_specs) and are quantised by the oracle's codec."""
    import synth
    from synth import workloads as W
    m = Model(shape)
    for spec in W.tensor_specs(shape, norm_jitter):
        if spec.fmt in (W.W4, W.I8):
            step = chunk_rows or max(1, (1 << 24) // spec.cols)
            for r0 in range(0, spec.rows, step):
                n = min(step, spec.rows - r0)
                w = synth.matrix_rows(spec, seed, r0, n)
                if spec.fmt == W.W4:
                    m.quant_w4_into(spec.layer, spec.kind, r0, w)
                else:
                    m.quant_lm_into(r0, w)
        elif spec.fmt == W.VEC:
            m.load_vec(spec.layer, spec.kind, synth.vector(spec, seed))
        elif spec.fmt == W.SIGNS:
            m.load_signs(synth.signs(spec.cols, seed, spec.stream))
        elif spec.fmt == W.MAP:
            m.set_draft_map(synth.draft_map(shape, seed))
    return m

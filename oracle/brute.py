"""Brute-force numpy model for tiny shapes (TEST INFRASTRUCTURE ONLY).

An independent second implementation of the decode step, written with the
literal matrix forms so that it can pin the C oracle:
  - Gated DeltaNet state update as the matrix product S (I - beta k k^T);
  - the randomized Hadamard transform as an explicit matrix from
    scipy.linalg.hadamard;
  - softmax from scipy.special, fp16 rounding from numpy's float16 cast.
The weights are the same logical codes and scales the C oracle holds.
"""
import numpy as np
from scipy.linalg import hadamard
from scipy.special import expit, softmax


def a16(x):
    """fp16 activation format, rounded from the fp32 value"""
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float16).astype(np.float64)


def f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def dequant_w4(codes, scales):
    codes = np.asarray(codes, np.uint8)
    lo = (codes & 15).astype(np.int64) - 8
    hi = (codes >> 4).astype(np.int64) - 8
    c = np.empty((codes.shape[0], codes.shape[1] * 2), np.int64)
    c[:, 0::2], c[:, 1::2] = lo, hi
    return c * np.repeat(f16(scales), 32, axis=1)


def dequant_i8(codes, scales):
    return np.asarray(codes, np.int64) * np.repeat(f16(scales), 32, axis=-1)


def quant(x, qmax):
    """group-32 symmetric RTN along the last axis, decisions in fp32"""
    x = np.asarray(x, np.float32)
    g = x.reshape(*x.shape[:-1], -1, 32)
    amax = np.abs(g).max(axis=-1, keepdims=True)
    s = (amax / np.float32(qmax)).astype(np.float16)
    sf = s.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.where(sf == 0, 0, np.clip(np.rint(g / sf), -qmax, qmax))
    return c.astype(np.int8).reshape(x.shape), s.view(np.uint16)[..., 0]


# Max's 8-level Gaussian quantizer (IRE Trans. Inf. Theory, 1960): output
# level magnitudes, rounded to fp16 for the cache
LM_MAGNITUDES = (0.2451, 0.7560, 1.3440, 2.1520)


def lm_levels():
    m = np.array(LM_MAGNITUDES, np.float32).astype(np.float16).astype(np.float64)
    return np.concatenate([-m[::-1], m])


def quant_lm(x):
    """Lloyd-Max group codec along the last axis (groups of 32): scale =
    fp16(sqrt(mean square)) with the mean square in fp32, code = index of the
    nearest level to x / scale (the lower one on a tie)"""
    x = np.asarray(x, np.float32)
    g = x.reshape(*x.shape[:-1], -1, 32)
    ms = np.mean(g.astype(np.float64) ** 2, axis=-1, keepdims=True).astype(np.float32)
    s = np.sqrt(ms).astype(np.float16)
    sf = s.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(sf == 0, 0, g / sf).astype(np.float32).astype(np.float64)
    lv = lm_levels()
    c = np.argmin(np.abs(t[..., None] - lv), axis=-1)
    c = np.where(sf == 0, 4, c)
    return c.astype(np.int8).reshape(x.shape), s.view(np.uint16)[..., 0]


def dequant_lm(codes, scales):
    return lm_levels()[np.asarray(codes, np.int64)] * np.repeat(f16(scales), 32, axis=-1)


def rmsnorm(x, w, eps):
    return x / np.sqrt(np.mean(x * x) + eps) * w


def silu(x):
    return x * expit(x)


class BruteModel:
    """weights: dict (layer, kind) -> array(s) in logical format, as loaded into the C oracle."""

    def __init__(self, shape, weights):
        self.s = shape
        self.w = weights
        self.pos = 0
        s = shape
        self.S = {}
        self.kv = {}
        for l, t in enumerate(s.pattern):
            if t == "G":
                self.S[l] = np.zeros((s.gdn_v_heads, s.gdn_head_dim, s.gdn_head_dim))
            else:
                self.kv[l] = []   # per position (kc, ks, vc, vs, fp16 k, fp16 rotated v), each [nkv][...]
        d = s.attn_head_dim
        self.dpos = 0
        if getattr(s, "draft_vocab", 0) > 0:
            self.kv[s.n_layers] = []     # the draft head's cache
        if "A" in s.pattern or getattr(s, "draft_vocab", 0) > 0:
            D = np.diag(weights[(-1, 11)].astype(np.float64))
            self.R = hadamard(d) @ D / np.sqrt(d)           # v' = R v
            self.Rinv = self.R.T                             # orthogonal

    def W(self, l, kind):
        c, sc = self.w[(l, kind)]
        return dequant_w4(c, sc)

    def gdn(self, l, xh):
        s = self.s
        nqk, nv, d = s.gdn_qk_heads, s.gdn_v_heads, s.gdn_head_dim
        p = self.W(l, 0) @ xh
        q = p[:nqk * d].reshape(nqk, d)
        k = p[nqk * d:2 * nqk * d].reshape(nqk, d)
        v = p[2 * nqk * d:2 * nqk * d + nv * d].reshape(nv, d)
        z = p[2 * nqk * d + nv * d:2 * nqk * d + 2 * nv * d].reshape(nv, d)
        a = p[2 * nqk * d + 2 * nv * d:2 * nqk * d + 2 * nv * d + nv]
        b = p[2 * nqk * d + 2 * nv * d + nv:]
        qn = q / np.sqrt((q * q).sum(1, keepdims=True) + s.rms_eps)
        kn = k / np.sqrt((k * k).sum(1, keepdims=True) + s.rms_eps)
        alpha = expit(a + self.w[(l, 9)])
        beta = expit(b)
        y = np.zeros((nv, d))
        for h in range(nv):
            j = h // (nv // nqk)
            kk = kn[j][:, None]
            S = self.S[l][h]
            S = alpha[h] * S @ (np.eye(d) - beta[h] * kk @ kk.T) + beta[h] * v[h][:, None] @ kk.T
            self.S[l][h] = S
            o = S @ qn[j]
            y[h] = a16(rmsnorm(o, self.w[(l, 8)], s.rms_eps) * silu(z[h]))
        return self.W(l, 1) @ y.ravel()

    def attn(self, l, xh):
        s = self.s
        nq, nkv, d = s.attn_q_heads, s.attn_kv_heads, s.attn_head_dim
        p = self.W(l, 0) @ xh
        q = p[:nq * d].reshape(nq, d)
        g = p[nq * d:2 * nq * d].reshape(nq, d)
        k = p[2 * nq * d:2 * nq * d + nkv * d].reshape(nkv, d)
        v = p[2 * nq * d + nkv * d:].reshape(nkv, d)
        fmt = getattr(s, "kv_format", 0)
        kc, ks = quant(k, 7 if fmt == 1 else 127)
        vr = v if fmt == 1 else (self.R @ v.T).T       # format 1 keeps values unrotated
        vc, vs = quant_lm(vr) if fmt == 2 else quant(vr, 7 if fmt == 1 else 3)
        vdq = dequant_lm if fmt == 2 else dequant_i8
        # the fp32 key and rotated value at fp16, for the recent window
        kh = k.astype(np.float32).astype(np.float16).astype(np.float64)
        vh = vr.astype(np.float32).astype(np.float16).astype(np.float64)
        self.kv[l].append((kc, ks, vc, vs, kh, vh))
        T = len(self.kv[l])
        win = getattr(s, "kv_window", 0) if l < s.n_layers else 0
        w0 = T - win if win > 0 else T          # positions w0.. are read at fp16
        K = np.stack([e[4] if t >= w0 else dequant_i8(e[0], e[1]) for t, e in enumerate(self.kv[l])])
        Vr = np.stack([e[5] if t >= w0 else vdq(e[2], e[3]) for t, e in enumerate(self.kv[l])])
        o = np.zeros((nq, d))
        for i in range(nq):
            j = i // (nq // nkv)
            sc = K[:, j, :] @ q[i] / np.sqrt(d)
            pr = softmax(sc)
            acc = pr @ Vr[:, j, :]
            o[i] = a16((acc if fmt == 1 else self.Rinv @ acc) * expit(g[i]))
        return self.W(l, 1) @ o.ravel()

    def block(self, l, t, x):
        s = self.s
        xh = a16(rmsnorm(x, self.w[(l, 6)], s.rms_eps))
        x = x + (self.gdn(l, xh) if t == "G" else self.attn(l, xh))
        xh = a16(rmsnorm(x, self.w[(l, 7)], s.rms_eps))
        h = a16(silu(self.W(l, 2) @ xh) * (self.W(l, 3) @ xh))
        return x + self.W(l, 4) @ h

    def forward_layers(self, x):
        x = np.array(x, np.float64)
        for l, t in enumerate(self.s.pattern):
            x = self.block(l, t, x)
        self.pos += 1
        return x

    def draft_step(self, token, h, slot=0):
        """Draft head on (token, h), weights at layer index n_layers: the
        concatenation [norm(embedding); norm(h)] through the fuse matrix, one
        gated-attention block whose cache keeps dpos + slot earlier entries, and
        the mapped rows of the int8 table (ids ascending) on the normalised
        output.  -> (output hidden, mapped logits)"""
        s = self.s
        D = s.n_layers
        u = np.concatenate([a16(rmsnorm(self.embed(token), self.w[(D, 13)], s.rms_eps)),
                            a16(rmsnorm(np.asarray(h, np.float64), self.w[(D, 14)], s.rms_eps))])
        x = self.W(D, 12) @ u
        del self.kv[D][self.dpos + slot:]
        x = self.block(D, "A", x)
        c, sc = self.w[(-1, 5)]
        ids = np.sort(np.asarray(self.w[(D, 16)]))
        z = dequant_i8(c[ids], sc[ids]) @ a16(rmsnorm(x, self.w[(D, 15)], s.rms_eps))
        return x, z

    def embed(self, token):
        c, sc = self.w[(-1, 5)]
        return dequant_i8(c[token], sc[token])

    def head(self, x):
        c, sc = self.w[(-1, 5)]
        xh = a16(rmsnorm(x, self.w[(-1, 10)], self.s.rms_eps))
        logits = dequant_i8(c, sc) @ xh
        return logits, int(np.argmax(logits))

    def decode_token(self, token):
        x = self.forward_layers(self.embed(token))
        logits, am = self.head(x)
        return x, logits, am

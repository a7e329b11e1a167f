"""Seeded synthetic inputs shared by the CPU oracle, the tests and the benchmark.

Two implementations of one generator definition (Philox4x32-10 + Irwin-Hall
normals, see synth_host.c): a host C library for the oracle and a device HIP
library that fills tensors directly in GPU memory.  Neither holds any of the
decode step's arithmetic.
"""
import ctypes
import os
import subprocess

import numpy as np

from . import workloads  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_SO = os.path.join(_HERE, "libaw4synth_host.so")
DEV_SO = os.path.join(_HERE, "libaw4synth_dev.so")
HIP_FLAGS = ["-O3", "--offload-arch=gfx950", "-fPIC", "-shared", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose=False):
    """Compile both generator libraries (host with gcc, device with hipcc)."""
    src_c = os.path.join(_HERE, "synth_host.c")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                           "-o", HOST_SO + ".tmp", src_c])
    os.replace(HOST_SO + ".tmp", HOST_SO)
    src_h = os.path.join(_HERE, "synth_dev.hip")
    subprocess.check_call(["hipcc", *HIP_FLAGS, "-o", DEV_SO + ".tmp", src_h],
                          stdout=None if verbose else subprocess.DEVNULL)
    os.replace(DEV_SO + ".tmp", DEV_SO)
    global _host, _dev
    _host = _dev = None


_host = None
_dev = None

_i64, _u64, _u32, _i32, _f32, _vp = (ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32,
                                     ctypes.c_int32, ctypes.c_float, ctypes.c_void_p)


def host():
    global _host
    if _host is None:
        if not os.path.exists(HOST_SO):
            raise RuntimeError(f"{HOST_SO} missing: run __graft_entry__.build()")
        L = ctypes.CDLL(HOST_SO)
        L.aw4s_philox4x32_10.argtypes = [_vp, _vp, _vp]
        L.aw4s_u32_at.argtypes = [_u64, _u32, _u64]
        L.aw4s_u32_at.restype = _u32
        L.aw4s_ih12_at.argtypes = [_u64, _u32, _u64]
        L.aw4s_ih12_at.restype = _i32
        L.aw4s_normal_f32.argtypes = [_vp, _i64, _i64, _i64, _f32, _u64, _u32]
        L.aw4s_one_plus_normal_f32.argtypes = [_vp, _i64, _f32, _u64, _u32]
        L.aw4s_u32.argtypes = [_vp, _i64, _i64, _u64, _u32]
        L.aw4s_uniform_f32.argtypes = [_vp, _i64, _i64, _u64, _u32]
        L.aw4s_tokens.argtypes = [_vp, _i64, _i64, _i32, _u64, _u32]
        L.aw4s_signs.argtypes = [_vp, _i64, _u64, _u32]
        L.aw4s_codes_i8.argtypes = [_vp, _i64, _i64, _i32, _i32, _u64, _u32]
        L.aw4s_scale_bits.argtypes = [_vp, _i64, _i64, ctypes.c_uint16, _u64, _u32]
        _host = L
    return _host


def dev():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_SO):
            raise RuntimeError(f"{DEV_SO} missing: run __graft_entry__.build()")
        import torch  # noqa: F401  (one HIP runtime: torch's, see attention_w4_amd.lib)
        L = ctypes.CDLL(DEV_SO)
        for n, a in [("aw4s_dev_normal_f32", [_vp, _i64, _i64, _i64, _f32, _u64, _u32, _vp]),
                     ("aw4s_dev_codes_i8", [_vp, _i64, _i64, _i32, _i32, _u64, _u32, _vp]),
                     ("aw4s_dev_scale_bits", [_vp, _i64, _i64, ctypes.c_uint16, _u64, _u32, _vp]),
                     ("aw4s_dev_u32", [_vp, _i64, _i64, _u64, _u32, _vp]),
                     ("aw4s_dev_tokens", [_vp, _i64, _i64, _i32, _u64, _u32, _vp])]:
            f = getattr(L, n)
            f.argtypes = a
            f.restype = ctypes.c_int
        _dev = L
    return _dev


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


# ------------------------------------------------------------------ host side
def philox(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    host().aw4s_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def normal(rows, cols, sigma, seed, stream, row0=0):
    out = np.empty((rows, cols), dtype=np.float32)
    host().aw4s_normal_f32(_ptr(out), row0, rows, cols, sigma, seed, stream)
    return out


def one_plus_normal(n, jitter, seed, stream):
    out = np.empty(n, dtype=np.float32)
    host().aw4s_one_plus_normal_f32(_ptr(out), n, jitter, seed, stream)
    return out


def u32(n, seed, stream, i0=0):
    out = np.empty(n, dtype=np.uint32)
    host().aw4s_u32(_ptr(out), i0, n, seed, stream)
    return out


def uniform(n, seed, stream, i0=0):
    out = np.empty(n, dtype=np.float32)
    host().aw4s_uniform_f32(_ptr(out), i0, n, seed, stream)
    return out


def tokens(n, vocab, seed, stream=workloads.STREAM_PROMPT, i0=0):
    out = np.empty(n, dtype=np.int32)
    host().aw4s_tokens(_ptr(out), i0, n, vocab, seed, stream)
    return out


def draft_map(shape, seed):
    """The draft head's vocabulary map: draft_vocab distinct ids drawn uniformly
    without replacement from [0, vocab) (the ids with the smallest of one
    Philox u32 key per id, ties broken by id), returned ascending."""
    keys = u32(shape.vocab, seed, workloads.STREAM_MAP).astype(np.uint64)
    order = np.argsort((keys << np.uint64(32)) | np.arange(shape.vocab, dtype=np.uint64), kind="stable")
    return np.sort(order[:shape.draft_vocab]).astype(np.int32)


def signs(n, seed, stream):
    out = np.empty(n, dtype=np.int8)
    host().aw4s_signs(_ptr(out), n, seed, stream)
    return out


def codes(n, spread256, qmax, seed, stream, i0=0):
    out = np.empty(n, dtype=np.int8)
    host().aw4s_codes_i8(_ptr(out), i0, n, spread256, qmax, seed, stream)
    return out


def scale_bits(n, base_bits, seed, stream, i0=0):
    out = np.empty(n, dtype=np.uint16)
    host().aw4s_scale_bits(_ptr(out), i0, n, base_bits, seed, stream)
    return out


def vector(spec, seed):
    """Values of a VEC tensor from the recipe."""
    if spec.const is not None:
        return np.full(spec.cols, spec.const, dtype=np.float32)
    return one_plus_normal(spec.cols, spec.jitter, seed, spec.stream)


def matrix_rows(spec, seed, row0, nrows):
    """fp32 rows [row0, row0+nrows) of a normal-filled matrix from the recipe."""
    out = np.empty((nrows, spec.cols), dtype=np.float32)
    for (a, b, sig) in spec.segments:
        lo, hi = max(a, row0), min(b, row0 + nrows)
        if lo < hi:
            host().aw4s_normal_f32(_ptr(out[lo - row0:]), lo, hi - lo, spec.cols, sig, seed, spec.stream)
    return out


# ------------------------------------------------------------------ device side
def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with hip error {rc}")


def dev_matrix_rows(out_ptr, spec, seed, row0, nrows, stream_ptr=None):
    """Fill fp32 rows [row0, row0+nrows) of a recipe matrix at device address out_ptr."""
    L = dev()
    for (a, b, sig) in spec.segments:
        lo, hi = max(a, row0), min(b, row0 + nrows)
        if lo < hi:
            _check(L.aw4s_dev_normal_f32(out_ptr + (lo - row0) * spec.cols * 4, lo, hi - lo,
                                         spec.cols, sig, seed, spec.stream, stream_ptr),
                   "aw4s_dev_normal_f32")


def dev_normal(out_ptr, rows, cols, sigma, seed, stream, row0=0, stream_ptr=None):
    _check(dev().aw4s_dev_normal_f32(out_ptr, row0, rows, cols, sigma, seed, stream, stream_ptr),
           "aw4s_dev_normal_f32")


def dev_codes(out_ptr, n, spread256, qmax, seed, stream, i0=0, stream_ptr=None):
    _check(dev().aw4s_dev_codes_i8(out_ptr, i0, n, spread256, qmax, seed, stream, stream_ptr),
           "aw4s_dev_codes_i8")


def dev_scale_bits(out_ptr, n, base_bits, seed, stream, i0=0, stream_ptr=None):
    _check(dev().aw4s_dev_scale_bits(out_ptr, i0, n, base_bits, seed, stream, stream_ptr),
           "aw4s_dev_scale_bits")


def dev_u32(out_ptr, n, seed, stream, i0=0, stream_ptr=None):
    _check(dev().aw4s_dev_u32(out_ptr, i0, n, seed, stream, stream_ptr), "aw4s_dev_u32")


def dev_tokens(out_ptr, n, vocab, seed, stream=workloads.STREAM_PROMPT, i0=0, stream_ptr=None):
    _check(dev().aw4s_dev_tokens(out_ptr, i0, n, vocab, seed, stream, stream_ptr), "aw4s_dev_tokens")

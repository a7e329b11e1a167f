"""Writer of the weight blob that aw4_load_weights reads (layout in
include/aw4.h, next to aw4_check_blob).

Serialisation only: every tensor arrives already in its logical format
(matrices as codes plus fp16 scale bits, vectors as fp32, the draft map as
int32 ids), so nothing here quantises or computes any part of the model.
"""
import struct

import numpy as np

MAGIC = b"AW4W"
VERSION = 4
SHAPE_FIELDS = ("hidden", "ffn", "vocab", "n_layers", "gdn_qk_heads", "gdn_v_heads", "gdn_head_dim",
                "attn_q_heads", "attn_kv_heads", "attn_head_dim", "group", "draft_vocab")
MATRIX_KINDS = (0, 1, 2, 3, 4, 5, 12)
LM_HEAD, DRAFT_MAP = 5, 16


def header(cfg, count):
    """magic, version, the config's shape fields, its layer pattern, tensor count"""
    pat = bytes(cfg.layer_pattern)
    return (MAGIC + struct.pack("<I", VERSION) +
            struct.pack("<12i", *[int(getattr(cfg, f)) for f in SHAPE_FIELDS]) +
            pat.ljust(128, b"\0")[:128] + struct.pack("<I", count))


def record(layer, kind, value):
    """(header, payload parts) of one tensor; value: (codes, scales) for a
    matrix kind, a 1-D array otherwise"""
    if kind in MATRIX_KINDS:
        codes, scales = value
        codes = np.ascontiguousarray(codes, np.int8 if kind == LM_HEAD else np.uint8)
        scales = np.ascontiguousarray(scales, np.uint16)
        rows, cols = scales.shape[0], scales.shape[1] * 32
        parts = [codes.tobytes(), scales.astype("<u2").tobytes()]
    else:
        arr = np.ascontiguousarray(value, np.int32 if kind == DRAFT_MAP else np.float32).ravel()
        rows, cols = 1, arr.size
        parts = [arr.astype("<i4" if kind == DRAFT_MAP else "<f4").tobytes()]
    nbytes = sum(len(p) for p in parts)
    return struct.pack("<iiqqQ", int(layer), int(kind), rows, cols, nbytes), parts


def write_blob(cfg, tensors, f=None):
    """Serialise tensors, an iterable of (layer, kind, value), for config cfg
    (an aw4_config structure).  Returns the blob as bytes, or writes it to the
    binary file object f and returns the byte count."""
    tensors = list(tensors)
    chunks = [header(cfg, len(tensors))]
    total = len(chunks[0])
    if f is not None:
        f.write(chunks[0])
    for layer, kind, value in tensors:
        h, parts = record(layer, kind, value)
        total += len(h) + sum(len(p) for p in parts)
        if f is not None:
            f.write(h)
            for p in parts:
                f.write(p)
        else:
            chunks.append(h)
            chunks.extend(parts)
    return total if f is not None else b"".join(chunks)

"""Test-side helpers written independently of the oracle and of the library.

They re-read the documented packed layout (token-major key rows; value codes
channel-major inside 64-token tiles) with NumPy, dequantize in binary64 and
evaluate plain softmax attention, so oracle pins do not lean on the oracle's
own unpacking code.
"""
from __future__ import annotations

import numpy as np


def unpack_k(codes: np.ndarray, bits: int, tq: int, D: int) -> np.ndarray:
    """codes [B][H][cap][D*bits/32] uint32 -> [B][H][tq][D] integer codes."""
    E = 32 // bits
    mask = (1 << bits) - 1
    d = np.arange(D)
    words = codes[:, :, :tq, d // E]                       # [B][H][tq][D]
    return ((words >> (bits * (d % E)).astype(np.uint32)) & mask).astype(np.int64)


def unpack_v(codes: np.ndarray, bits: int, tq: int, D: int) -> np.ndarray:
    """codes [B][H][cap/64][D][64*bits/32] -> [B][H][tq][D] integer codes."""
    E = 32 // bits
    mask = (1 << bits) - 1
    t = np.arange(tq)
    tile, tau = t // 64, t % 64
    w = codes[:, :, tile, :, :]                              # [B][H][tq][D][WPC]
    w = np.take_along_axis(w, (tau // E)[None, None, :, None, None].repeat(D, 3), axis=4)[..., 0]
    shift = (bits * (tau % E)).astype(np.uint32)[None, None, :, None]
    return ((w >> shift) & mask).astype(np.int64)


def dequant_k(codes, scale, zero, bits, G, tq, D):
    c = unpack_k(codes, bits, tq, D).astype(np.float64)
    s = np.repeat(scale.astype(np.float64), G, axis=2)[:, :, :tq]
    z = np.repeat(zero.astype(np.float64), G, axis=2)[:, :, :tq]
    return c * s + z


def dequant_v(codes, scale, zero, bits, G, tq, D):
    c = unpack_v(codes, bits, tq, D).astype(np.float64)
    s = np.repeat(scale.astype(np.float64)[:, :, :tq], G, axis=3)
    z = np.repeat(zero.astype(np.float64)[:, :, :tq], G, axis=3)
    return c * s + z


def attention_f64(q, k, v, scale):
    """Plain softmax attention.  q [B][Hq][D], k/v [B][Hkv][T][D] (any float
    dtype), query head h reads kv head h // (Hq/Hkv).  Returns float64."""
    q = q.astype(np.float64)
    k = k.astype(np.float64)
    v = v.astype(np.float64)
    r = q.shape[1] // k.shape[1]
    k = np.repeat(k, r, axis=1)
    v = np.repeat(v, r, axis=1)
    logits = np.einsum("bhd,bhtd->bht", q, k) * float(scale)
    logits -= logits.max(axis=2, keepdims=True)
    p = np.exp(logits)
    return np.einsum("bht,bhtd->bhd", p, v) / p.sum(axis=2)[..., None]


def row_rel_err(o_test, o_ref):
    """Per (b, h) row: max_d |o_test - o_ref| / max_d |o_ref|; returns the max
    over rows."""
    o_test = np.asarray(o_test, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    num = np.abs(o_test - o_ref).max(axis=-1)
    den = np.abs(o_ref).max(axis=-1)
    return float((num / np.maximum(den, 1e-30)).max())

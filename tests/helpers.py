"""Test-side helpers written independently of the oracle and of the library.

They re-read the documented packed layout (token-major key rows; value codes
channel-major inside 64-token tiles; the per-width bit orders) with NumPy, dequantize in binary64 and
evaluate plain softmax attention, so oracle pins do not lean on the oracle's
own unpacking code.
"""
from __future__ import annotations

import numpy as np


def beta(p):
    """Bit of position p (0..31) inside a one-bit code word: 4*((p%16)//2) +
    2*(p//16) + p%2 (the documented one-bit order)."""
    p = np.asarray(p)
    return 4 * ((p % 16) // 2) + 2 * (p // 16) + p % 2


def row_codes(rows: np.ndarray, bits: int, n: int, pos: np.ndarray) -> np.ndarray:
    """Codes at positions ``pos`` of rows of n codes (rows: [..., n*bits/32]
    uint32 words; pos broadcast against the leading axes) per the documented
    layouts: b = 2, 4 little-endian E = 32/b per word; b = 1 at bit beta(p%32)
    of word p/32; b = 3 a two-bit plane (word p/16, bits 2*(p%16)) followed
    by a one-bit plane of the high bit (word n/16 + p/32, bit beta(p%32))."""
    rows = rows.astype(np.int64)
    pos = np.asarray(pos)

    def word(i):
        return np.take_along_axis(rows, np.broadcast_to(i, rows.shape[:-1])[..., None], -1)[..., 0]

    if bits == 3:
        lo = (word(pos // 16) >> (2 * (pos % 16))) & 3
        hi = (word(n // 16 + pos // 32) >> beta(pos % 32)) & 1
        return lo | (hi << 2)
    if bits == 1:
        return (word(pos // 32) >> beta(pos % 32)) & 1
    E = 32 // bits
    return (word(pos // E) >> (bits * (pos % E))) & ((1 << bits) - 1)


def unpack_k(codes: np.ndarray, bits: int, tq: int, D: int) -> np.ndarray:
    """codes [B][H][cap][D*bits/32] uint32 -> [B][H][tq][D] integer codes."""
    rows = codes[:, :, :tq, None, :]                      # [B][H][tq][1][W]
    rows = np.broadcast_to(rows, rows.shape[:3] + (D, rows.shape[-1]))
    return row_codes(rows, bits, D, np.arange(D)[None, None, None, :])


def unpack_v(codes: np.ndarray, bits: int, tq: int, D: int) -> np.ndarray:
    """codes [B][H][cap/64][D][2*bits] -> [B][H][tq][D] integer codes."""
    t = np.arange(tq)
    rows = codes[:, :, t // 64, :, :]                     # [B][H][tq][D][WPC]
    return row_codes(rows, bits, 64, (t % 64)[None, None, :, None])


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


def unpack_outliers(outl: np.ndarray):
    """Key-outlier store [B][H][cap/G][n_out][D] uint32 -> (positions, values):
    positions inside the group (word >> 16) and binary16 values (low half),
    both [B][H][cap/G][n_out][D] (the documented word format)."""
    w = outl.astype(np.uint32)
    pos = (w >> 16).astype(np.int64)
    val = (w & 0xFFFF).astype(np.uint16).view(np.float16)
    return pos, val


def dequant_k_sparse(codes, scale, zero, outl, bits, G, tq, D):
    """Dense dequantization, then every listed outlier (group g, channel d,
    position i) replaces the value of token g*G + i, channel d."""
    k = dequant_k(codes, scale, zero, bits, G, tq, D)
    if outl is None:
        return k
    pos, val = unpack_outliers(outl)
    B, H, NGk, n_out, _ = outl.shape
    for g in range(tq // G):
        for j in range(n_out):
            t = g * G + pos[:, :, g, j, :]                       # [B][H][D]
            bi, hi, di = np.meshgrid(np.arange(B), np.arange(H), np.arange(D), indexing="ij")
            k[bi, hi, t, di] = val[:, :, g, j, :].astype(np.float64)
    return k


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

"""KiviCache: device buffers for one layer's mixed-precision KV cache.

PyTorch only allocates the buffers and supplies the current HIP stream; all
computation goes through the C ABI (``_lib``) into the HIP kernels.
"""
from __future__ import annotations

import ctypes

import torch

import numpy as np

from . import _lib
from ._lib import check, kivi_cache, kivi_paged_cache, kivi_ragged_cache, kivi_shape


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def make_shape(batch, kv_heads, gqa, head_dim, bits, group, residual, capacity,
               meta_half=False, outliers=0, rope_theta=0.0, deterministic=False,
               v_window=False) -> kivi_shape:
    return kivi_shape(batch, kv_heads, gqa, head_dim, bits, group, residual, capacity,
                      int(bool(meta_half)), int(outliers), float(rope_theta),
                      int(bool(deterministic)), int(bool(v_window)))


def _outlier_store(shape: kivi_shape, lead: int, tokens: int, page_tokens: int, num_pages: int,
                   dev) -> torch.Tensor | None:
    """Key-outlier store [lead][H][tokens/G][n][D] (int32 words), or None."""
    n = shape.outliers
    if n == 0:
        return None
    nbytes = ctypes.c_size_t()
    check(_lib.kivi_outlier_bytes(ctypes.byref(shape), page_tokens, num_pages,
                                  ctypes.byref(nbytes)), "kivi_outlier_bytes")
    t = torch.zeros((lead, shape.num_kv_heads, tokens // shape.group, n, shape.head_dim),
                    dtype=torch.int32, device=dev)
    assert t.nbytes == nbytes.value
    return t


class KiviCache:
    """One layer's cache: packed K/V codes, scale/zero (fp32, or fp16 when
    meta_half), fp16 residual, and with ``outliers`` > 0 the key-outlier
    store (that many kept keys per key group and channel); with
    ``rope_theta`` > 0 the keys are pre-RoPE and decode rotates them; with
    ``deterministic`` repeated decodes give identical bits (by default the
    waves of a block share its tiles in load-return order); with
    ``v_window`` the values keep a sliding window of the ``residual`` newest
    tokens in full precision (v_res slot t % residual) and are quantized one
    token at a time as they leave it.

    Layouts are those of include/kivi.h; the host keeps (tq, tr)."""

    def __init__(self, batch, kv_heads, gqa, head_dim, bits, group, residual, capacity,
                 device="cuda", meta_half=False, outliers=0, rope_theta=0.0,
                 deterministic=False, v_window=False):
        self.shape = make_shape(batch, kv_heads, gqa, head_dim, bits, group, residual, capacity,
                                meta_half, outliers, rope_theta, deterministic, v_window)
        self.meta_half = bool(meta_half)
        self.outliers = int(outliers)
        mdt = torch.float16 if meta_half else torch.float32
        sizes = [ctypes.c_size_t() for _ in range(6)]
        check(_lib.kivi_cache_bytes(ctypes.byref(self.shape), *[ctypes.byref(s) for s in sizes]),
              "kivi_cache_bytes")
        B, H, D, G, R, cap = batch, kv_heads, head_dim, group, residual, capacity
        dev = torch.device(device)
        self.k_codes = torch.zeros((B, H, cap, D * bits // 32), dtype=torch.int32, device=dev)
        self.k_scale = torch.zeros((B, H, cap // G, D), dtype=mdt, device=dev)
        self.k_zero = torch.zeros((B, H, cap // G, D), dtype=mdt, device=dev)
        self.v_codes = torch.zeros((B, H, cap // 64, D, 2 * bits), dtype=torch.int32, device=dev)
        self.v_scale = torch.zeros((B, H, cap, D // G), dtype=mdt, device=dev)
        self.v_zero = torch.zeros((B, H, cap, D // G), dtype=mdt, device=dev)
        self.k_res = torch.zeros((B, H, R, D), dtype=torch.float16, device=dev)
        self.v_res = torch.zeros((B, H, R, D), dtype=torch.float16, device=dev)
        assert self.k_codes.numel() * 4 == sizes[0].value
        assert self.k_scale.nbytes == sizes[1].value
        assert self.v_codes.numel() * 4 == sizes[2].value
        assert self.v_scale.nbytes == sizes[3].value
        assert self.k_res.numel() * 2 == sizes[4].value
        self.k_outliers = _outlier_store(self.shape, B, cap, 0, 0, dev)
        self.c = kivi_cache(self.shape, *[t.data_ptr() for t in (
            self.k_codes, self.k_scale, self.k_zero, self.v_codes, self.v_scale, self.v_zero,
            self.k_res, self.v_res)], 0, 0, _ptr(self.k_outliers))
        self.workspace = None

    # lengths live on the host, inside the C struct
    @property
    def tq(self) -> int:
        return self.c.tq

    @property
    def tr(self) -> int:
        return self.c.tr

    def set_lengths(self, tq: int, tr: int) -> None:
        self.c.tq, self.c.tr = tq, tr

    def prefill(self, k: torch.Tensor, v: torch.Tensor, tq: int) -> None:
        """k, v: fp16 [B][Hkv][T][D] contiguous device tensors."""
        assert k.dtype == torch.float16 and k.is_contiguous() and v.is_contiguous()
        check(_lib.kivi_prefill(ctypes.byref(self.c), k.data_ptr(), v.data_ptr(), k.shape[2], tq,
                                _stream()), "kivi_prefill")

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor) -> None:
        """k_new, v_new: fp16 [B][Hkv][D]."""
        assert k_new.is_contiguous() and v_new.is_contiguous()
        check(_lib.kivi_append(ctypes.byref(self.c), k_new.data_ptr(), v_new.data_ptr(),
                               _stream()), "kivi_append")

    def workspace_for(self, num_splits: int = 0) -> torch.Tensor | None:
        nbytes = _lib.kivi_decode_workspace_bytes(ctypes.byref(self.shape), num_splits)
        if nbytes == 0:
            return None
        if self.workspace is None or self.workspace.numel() < nbytes:
            self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.k_codes.device)
        return self.workspace

    def decode(self, q: torch.Tensor, softmax_scale: float, out: torch.Tensor | None = None,
               num_splits: int = 0) -> torch.Tensor:
        """q: fp16 [B][Hkv*r][D] -> fp16 output of the same shape."""
        assert q.dtype == torch.float16 and q.is_contiguous()
        if out is None:
            out = torch.empty_like(q)
        ws = self.workspace_for(num_splits)
        nb = 0 if ws is None else ws.numel()
        check(_lib.kivi_decode_attn(ctypes.byref(self.c), q.data_ptr(), float(softmax_scale),
                                    out.data_ptr(), _ptr(ws), nb, num_splits, _stream()),
              "kivi_decode_attn")
        return out

    def append_decode(self, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                      softmax_scale: float, out: torch.Tensor | None = None,
                      num_splits: int = 0) -> torch.Tensor:
        """append(k_new, v_new) then decode(q) in one C call (one launch where
        the matrix-core kernel applies)."""
        assert k_new.is_contiguous() and v_new.is_contiguous()
        assert q.dtype == torch.float16 and q.is_contiguous()
        if out is None:
            out = torch.empty_like(q)
        ws = self.workspace_for(num_splits)
        nb = 0 if ws is None else ws.numel()
        check(_lib.kivi_append_decode_attn(ctypes.byref(self.c), k_new.data_ptr(),
                                           v_new.data_ptr(), q.data_ptr(), float(softmax_scale),
                                           out.data_ptr(), _ptr(ws), nb, num_splits, _stream()),
              "kivi_append_decode_attn")
        return out

    def auto_splits(self) -> int:
        s = _lib.kivi_decode_auto_splits(ctypes.byref(self.c))
        if s < 0:
            check(-s, "kivi_decode_auto_splits")
        return s


def quantize_k(shape: kivi_shape, k: torch.Tensor, ntok: int, dst_off: int, codes, scale, zero,
               outliers: torch.Tensor | None = None):
    """kivi_quantize_k, or kivi_quantize_k_outliers when shape.outliers > 0."""
    if shape.outliers > 0:
        check(_lib.kivi_quantize_k_outliers(
            ctypes.byref(shape), k.data_ptr(), k.shape[2], ntok, dst_off, codes.data_ptr(),
            scale.data_ptr(), zero.data_ptr(), _ptr(outliers), _stream()),
            "kivi_quantize_k_outliers")
        return
    check(_lib.kivi_quantize_k(ctypes.byref(shape), k.data_ptr(), k.shape[2], ntok, dst_off,
                               codes.data_ptr(), scale.data_ptr(), zero.data_ptr(), _stream()),
          "kivi_quantize_k")


def quantize_v(shape: kivi_shape, v: torch.Tensor, ntok: int, dst_off: int, codes, scale, zero):
    check(_lib.kivi_quantize_v(ctypes.byref(shape), v.data_ptr(), v.shape[2], ntok, dst_off,
                               codes.data_ptr(), scale.data_ptr(), zero.data_ptr(), _stream()),
          "kivi_quantize_v")


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


class RaggedKiviCache(KiviCache):
    """A batch whose sequences have their own lengths: the same device
    buffers as KiviCache, per-sequence host length arrays ``tq``, ``tr``
    (int32 NumPy arrays the C struct points at; the library updates them)."""

    def __init__(self, batch, kv_heads, gqa, head_dim, bits, group, residual, capacity,
                 device="cuda", meta_half=False, outliers=0, rope_theta=0.0,
                 deterministic=False):
        super().__init__(batch, kv_heads, gqa, head_dim, bits, group, residual, capacity,
                         device=device, meta_half=meta_half, outliers=outliers,
                         rope_theta=rope_theta, deterministic=deterministic)
        self.tq_arr = np.zeros(batch, np.int32)
        self.tr_arr = np.zeros(batch, np.int32)
        self.rc = kivi_ragged_cache(self.shape, *[t.data_ptr() for t in (
            self.k_codes, self.k_scale, self.k_zero, self.v_codes, self.v_scale, self.v_zero,
            self.k_res, self.v_res)], _i32p(self.tq_arr), _i32p(self.tr_arr),
            _ptr(self.k_outliers))

    @property
    def tq(self) -> np.ndarray:
        return self.tq_arr.copy()

    @property
    def tr(self) -> np.ndarray:
        return self.tr_arr.copy()

    def set_lengths(self, tq, tr) -> None:
        self.tq_arr[:] = tq
        self.tr_arr[:] = tr

    def prefill(self, k: torch.Tensor, v: torch.Tensor, ntok, tq) -> None:
        """k, v: fp16 [B][Hkv][T][D]; sequence b uses its first ntok[b] tokens,
        the first tq[b] of them quantized."""
        assert k.dtype == torch.float16 and k.is_contiguous() and v.is_contiguous()
        n = np.ascontiguousarray(ntok, np.int32)
        t = np.ascontiguousarray(tq, np.int32)
        check(_lib.kivi_ragged_prefill(ctypes.byref(self.rc), k.data_ptr(), v.data_ptr(),
                                       k.shape[2], _i32p(n), _i32p(t), _stream()),
              "kivi_ragged_prefill")

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor) -> None:
        assert k_new.is_contiguous() and v_new.is_contiguous()
        check(_lib.kivi_ragged_append(ctypes.byref(self.rc), k_new.data_ptr(), v_new.data_ptr(),
                                      _stream()), "kivi_ragged_append")

    def decode(self, q: torch.Tensor, softmax_scale: float, out: torch.Tensor | None = None,
               num_splits: int = 0) -> torch.Tensor:
        assert q.dtype == torch.float16 and q.is_contiguous()
        if out is None:
            out = torch.empty_like(q)
        ws = self.workspace_for(num_splits)
        nb = 0 if ws is None else ws.numel()
        check(_lib.kivi_ragged_decode_attn(ctypes.byref(self.rc), q.data_ptr(),
                                           float(softmax_scale), out.data_ptr(), _ptr(ws), nb,
                                           num_splits, _stream()), "kivi_ragged_decode_attn")
        return out

    def append_decode(self, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                      softmax_scale: float, out: torch.Tensor | None = None,
                      num_splits: int = 0) -> torch.Tensor:
        assert k_new.is_contiguous() and v_new.is_contiguous()
        assert q.dtype == torch.float16 and q.is_contiguous()
        if out is None:
            out = torch.empty_like(q)
        ws = self.workspace_for(num_splits)
        nb = 0 if ws is None else ws.numel()
        check(_lib.kivi_ragged_append_decode_attn(
            ctypes.byref(self.rc), k_new.data_ptr(), v_new.data_ptr(), q.data_ptr(),
            float(softmax_scale), out.data_ptr(), _ptr(ws), nb, num_splits, _stream()),
            "kivi_ragged_append_decode_attn")
        return out

    def auto_splits(self) -> int:
        s = _lib.kivi_ragged_decode_auto_splits(ctypes.byref(self.rc))
        if s < 0:
            check(-s, "kivi_ragged_decode_auto_splits")
        return s


class PagedKiviCache(RaggedKiviCache):
    """A ragged batch whose quantized tokens live in page pools.

    ``table`` (int32 [batch][capacity // page_tokens], host array) names the
    page of every logical page of every sequence; it is copied to a device
    tensor (``self.table``).  By default sequence b's j-th page is page
    b * (capacity // page_tokens) + j.  Pools have the layouts of
    include/kivi.h; the residual stays per sequence."""

    def __init__(self, batch, kv_heads, gqa, head_dim, bits, group, residual, capacity,
                 page_tokens, num_pages=None, table=None, device="cuda", meta_half=False,
                 outliers=0, rope_theta=0.0, deterministic=False):
        self.shape = make_shape(batch, kv_heads, gqa, head_dim, bits, group, residual, capacity,
                                meta_half, outliers, rope_theta, deterministic)
        self.meta_half = bool(meta_half)
        self.outliers = int(outliers)
        P = page_tokens
        max_pages = capacity // P
        if num_pages is None:
            num_pages = batch * max_pages
        sizes = [ctypes.c_size_t() for _ in range(4)]
        check(_lib.kivi_paged_pool_bytes(ctypes.byref(self.shape), P, num_pages,
                                         *[ctypes.byref(x) for x in sizes]),
              "kivi_paged_pool_bytes")
        B, H, D, G, R = batch, kv_heads, head_dim, group, residual
        dev = torch.device(device)
        mdt = torch.float16 if meta_half else torch.float32
        self.page_tokens, self.num_pages, self.max_pages = P, num_pages, max_pages
        self.k_codes = torch.zeros((num_pages, H, P, D * bits // 32), dtype=torch.int32, device=dev)
        self.k_scale = torch.zeros((num_pages, H, P // G, D), dtype=mdt, device=dev)
        self.k_zero = torch.zeros((num_pages, H, P // G, D), dtype=mdt, device=dev)
        self.v_codes = torch.zeros((num_pages, H, P // 64, D, 2 * bits), dtype=torch.int32,
                                   device=dev)
        self.v_scale = torch.zeros((num_pages, H, P, D // G), dtype=mdt, device=dev)
        self.v_zero = torch.zeros((num_pages, H, P, D // G), dtype=mdt, device=dev)
        self.k_res = torch.zeros((B, H, R, D), dtype=torch.float16, device=dev)
        self.v_res = torch.zeros((B, H, R, D), dtype=torch.float16, device=dev)
        assert self.k_codes.nbytes == sizes[0].value and self.k_scale.nbytes == sizes[1].value
        assert self.v_codes.nbytes == sizes[2].value and self.v_scale.nbytes == sizes[3].value
        self.k_outliers = _outlier_store(self.shape, num_pages, P, P, num_pages, dev)
        if table is None:
            table = np.arange(B * max_pages, dtype=np.int32).reshape(B, max_pages)
        self.table_host = np.ascontiguousarray(table, np.int32).reshape(B, max_pages)
        self.table = torch.from_numpy(self.table_host.copy()).to(dev)
        self.tq_arr = np.zeros(batch, np.int32)
        self.tr_arr = np.zeros(batch, np.int32)
        self.pc = kivi_paged_cache(self.shape, P, num_pages, *[t.data_ptr() for t in (
            self.k_codes, self.k_scale, self.k_zero, self.v_codes, self.v_scale, self.v_zero,
            self.k_res, self.v_res, self.table)], _i32p(self.tq_arr), _i32p(self.tr_arr),
            _ptr(self.k_outliers))
        self.workspace = None

    def prefill(self, k, v, ntok, tq) -> None:
        assert k.dtype == torch.float16 and k.is_contiguous() and v.is_contiguous()
        n = np.ascontiguousarray(ntok, np.int32)
        t = np.ascontiguousarray(tq, np.int32)
        check(_lib.kivi_paged_prefill(ctypes.byref(self.pc), k.data_ptr(), v.data_ptr(),
                                      k.shape[2], _i32p(n), _i32p(t), _stream()),
              "kivi_paged_prefill")

    def append(self, k_new, v_new) -> None:
        assert k_new.is_contiguous() and v_new.is_contiguous()
        check(_lib.kivi_paged_append(ctypes.byref(self.pc), k_new.data_ptr(), v_new.data_ptr(),
                                     _stream()), "kivi_paged_append")

    def decode(self, q, softmax_scale, out=None, num_splits=0):
        assert q.dtype == torch.float16 and q.is_contiguous()
        if out is None:
            out = torch.empty_like(q)
        ws = self.workspace_for(num_splits)
        nb = 0 if ws is None else ws.numel()
        check(_lib.kivi_paged_decode_attn(ctypes.byref(self.pc), q.data_ptr(),
                                          float(softmax_scale), out.data_ptr(), _ptr(ws), nb,
                                          num_splits, _stream()), "kivi_paged_decode_attn")
        return out

    def append_decode(self, k_new, v_new, q, softmax_scale, out=None, num_splits=0):
        assert k_new.is_contiguous() and v_new.is_contiguous()
        assert q.dtype == torch.float16 and q.is_contiguous()
        if out is None:
            out = torch.empty_like(q)
        ws = self.workspace_for(num_splits)
        nb = 0 if ws is None else ws.numel()
        check(_lib.kivi_paged_append_decode_attn(
            ctypes.byref(self.pc), k_new.data_ptr(), v_new.data_ptr(), q.data_ptr(),
            float(softmax_scale), out.data_ptr(), _ptr(ws), nb, num_splits, _stream()),
            "kivi_paged_append_decode_attn")
        return out

    def auto_splits(self) -> int:
        s = _lib.kivi_paged_decode_auto_splits(ctypes.byref(self.pc))
        if s < 0:
            check(-s, "kivi_paged_decode_auto_splits")
        return s

    def gather(self, name: str) -> np.ndarray:
        """Host copy of a quantized-store buffer in the contiguous layout
        ([batch][H][capacity-derived axis]...), assembled from the pages named
        by the table (logical pages with an entry outside the pool are zero)."""
        pool = getattr(self, name).cpu().numpy()
        B, mp = self.table_host.shape
        parts = []
        for b in range(B):
            row = []
            for j in range(mp):
                pg = int(self.table_host[b, j])
                row.append(pool[pg] if 0 <= pg < self.num_pages else np.zeros_like(pool[0]))
            parts.append(np.concatenate(row, axis=1))
        return np.stack(parts)

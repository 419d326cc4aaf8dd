"""ctypes marshalling for the C oracle (test infrastructure only).

Every function here converts NumPy arrays to pointers and calls one function
of ``kivi_oracle.c``; none of the method's arithmetic is done in Python.
Array layouts are the ones documented at the top of ``kivi_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kivi_oracle.c")
_LIB = os.path.join(_HERE, "libkivi_oracle.so")
_CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11", "-Wall",
           "-Wextra", "-shared", "-fPIC"]

_lib = None

_u16p = ctypes.POINTER(ctypes.c_uint16)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int)
_vp = ctypes.c_void_p
_int = ctypes.c_int

ERRORS = {0: "ok", 1: "EINVAL", 2: "ESHAPE", 3: "ECAPACITY"}


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile kivi_oracle.c with gcc into libkivi_oracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    lib.kivio_half_to_float.argtypes = [ctypes.c_uint16]
    lib.kivio_half_to_float.restype = ctypes.c_float
    lib.kivio_float_to_half.argtypes = [ctypes.c_float]
    lib.kivio_float_to_half.restype = ctypes.c_uint16
    q_args = [_int] * 7 + [_u16p, _int, _int, _int, _u32p, _vp, _vp]
    lib.kivio_quantize_k.argtypes = q_args + [_int, _u32p]
    lib.kivio_quantize_v.argtypes = q_args
    lib.kivio_quantize_k.restype = _int
    lib.kivio_quantize_v.restype = _int
    lib.kivio_append.argtypes = [_int] * 8 + [_u32p, _vp, _vp, _u32p, _vp, _vp,
                                             _u16p, _u16p, _u16p, _u16p, _i32p, _i32p,
                                             _int, _u32p]
    lib.kivio_append.restype = _int
    lib.kivio_append_vw.argtypes = lib.kivio_append.argtypes
    lib.kivio_append_vw.restype = _int
    lib.kivio_quantize_v_token.argtypes = [_int] * 7 + [_u16p, _int, _int, _int, _u32p, _vp,
                                                        _vp]
    lib.kivio_quantize_v_token.restype = _int
    lib.kivio_decode_attn.argtypes = [_int] * 9 + [_u32p, _vp, _vp, _u32p, _vp,
                                                   _vp, _u16p, _u16p, _int, _int, _u16p,
                                                   ctypes.c_float, _f64p, _f64p, _int, _u32p,
                                                   ctypes.c_double]
    lib.kivio_decode_attn.restype = _int
    lib.kivio_decode_attn_vw.argtypes = lib.kivio_decode_attn.argtypes + [_int]
    lib.kivio_decode_attn_vw.restype = _int
    _lib = lib
    return lib


def _p(a: np.ndarray, ctype, dtype):
    assert a.dtype == dtype, (a.dtype, dtype)
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _m(a: np.ndarray, meta_half: bool):
    """Metadata array pointer: binary32, or binary16 bits (uint16) when meta_half."""
    assert a.dtype == (np.uint16 if meta_half else np.float32), a.dtype
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_vp)


def meta_dtype(meta_half: bool):
    return np.uint16 if meta_half else np.float32


def _h(a):  # binary16 bits, as uint16 (accepts float16 arrays too)
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    return a


def _check(rc):
    if rc != 0:
        raise OracleError(ERRORS.get(rc, str(rc)))


def half_to_float(bits: int) -> float:
    return float(load().kivio_half_to_float(int(bits)))


def float_to_half(x: float) -> int:
    """binary32 -> binary16 bits, round to nearest even (the oracle's own)."""
    return int(load().kivio_float_to_half(float(x)))


def code_words_k(cap: int, D: int, bits: int) -> int:
    return cap * D * bits // 32


def _quantize(fn, x, bits, G, cap, ntok, dst_off, codes, scale, zero, meta_half, *extra):
    x = _h(x)
    B, H, in_stride, D = x.shape
    _check(fn(B, H, D, bits, G, cap, int(meta_half), _p(x, ctypes.c_uint16, np.uint16),
              in_stride, ntok, dst_off, _p(codes, ctypes.c_uint32, np.uint32),
              _m(scale, meta_half), _m(zero, meta_half), *extra))


def _outl(a):
    """Pointer to a key-outlier array, or NULL."""
    return None if a is None else _p(a, ctypes.c_uint32, np.uint32)


def outlier_shape(B, H, cap, G, n_out, D):
    """Key-outlier store [B][H][cap/G][n_out][D] (uint32 words)."""
    return (B, H, cap // G, n_out, D)


def quantize_k(k, bits, G, cap, ntok=None, dst_off=0, codes=None, scale=None, zero=None,
               meta_half=False, n_out=0, outl=None):
    """Quantize keys k[B][H][T][D] (binary16) tokens [0, ntok) into a store of
    capacity cap at token offset dst_off.  Returns (codes, scale, zero); scale
    and zero are binary32, or binary16 bits (uint16) when meta_half.  With
    n_out > 0 each key group's n_out outliers go to ``outl`` (allocated when
    None; returned as a fourth element)."""
    k = _h(k)
    B, H, T, D = k.shape
    ntok = T if ntok is None else ntok
    if codes is None:
        codes = np.zeros((B, H, cap, D * bits // 32), np.uint32)
        scale = np.zeros((B, H, cap // G, D), meta_dtype(meta_half))
        zero = np.zeros((B, H, cap // G, D), meta_dtype(meta_half))
    if n_out and outl is None:
        outl = np.zeros(outlier_shape(B, H, cap, G, n_out, D), np.uint32)
    _quantize(load().kivio_quantize_k, k, bits, G, cap, ntok, dst_off, codes, scale, zero,
              meta_half, int(n_out), _outl(outl if n_out else None))
    if n_out:
        return codes, scale, zero, outl
    return codes, scale, zero


def quantize_v(v, bits, G, cap, ntok=None, dst_off=0, codes=None, scale=None, zero=None,
               meta_half=False):
    """Quantize values v[B][H][T][D] (binary16).  Returns (codes, scale, zero)
    with codes in the 64-token channel-major tile layout."""
    v = _h(v)
    B, H, T, D = v.shape
    ntok = T if ntok is None else ntok
    if codes is None:
        codes = np.zeros((B, H, cap // 64, D, 64 * bits // 32), np.uint32)
        scale = np.zeros((B, H, cap, D // G), meta_dtype(meta_half))
        zero = np.zeros((B, H, cap, D // G), meta_dtype(meta_half))
    _quantize(load().kivio_quantize_v, v, bits, G, cap, ntok, dst_off, codes, scale, zero,
              meta_half)
    return codes, scale, zero


def quantize_v_token(v, slot, t, bits, G, cap, codes, scale, zero, meta_half=False):
    """Quantize source row ``slot`` of v[B][H][S][D] (binary16) as cache token
    t of the value store (codes, scale, zero updated in place)."""
    v = _h(v)
    B, H, S, D = v.shape
    _check(load().kivio_quantize_v_token(
        B, H, D, bits, G, cap, int(meta_half), _p(v, ctypes.c_uint16, np.uint16), S, slot, t,
        _p(codes, ctypes.c_uint32, np.uint32), _m(scale, meta_half), _m(zero, meta_half)))


@dataclass
class OracleCache:
    """Host-side mixed-precision cache driven by the C oracle."""
    B: int
    H: int
    r: int
    D: int
    bits: int
    G: int
    R: int
    cap: int
    meta_half: bool = False
    n_out: int = 0          # key outliers per key group (0: none)
    rope_theta: float = 0.0  # > 0: keys are pre-RoPE, rotated at decode (base rope_theta)
    v_window: bool = False   # values: a sliding window of the R newest tokens (v_res slot t % R)
    tq: int = 0
    tr: int = 0
    k_codes: np.ndarray = field(default=None, repr=False)
    ks: np.ndarray = field(default=None, repr=False)
    kz: np.ndarray = field(default=None, repr=False)
    v_codes: np.ndarray = field(default=None, repr=False)
    vs: np.ndarray = field(default=None, repr=False)
    vz: np.ndarray = field(default=None, repr=False)
    k_res: np.ndarray = field(default=None, repr=False)
    v_res: np.ndarray = field(default=None, repr=False)
    k_outl: np.ndarray = field(default=None, repr=False)
    flushes: int = 0

    def __post_init__(self):
        B, H, D, bits, G, R, cap = self.B, self.H, self.D, self.bits, self.G, self.R, self.cap
        md = meta_dtype(self.meta_half)
        self.k_codes = np.zeros((B, H, cap, D * bits // 32), np.uint32)
        self.ks = np.zeros((B, H, cap // G, D), md)
        self.kz = np.zeros((B, H, cap // G, D), md)
        self.v_codes = np.zeros((B, H, cap // 64, D, 64 * bits // 32), np.uint32)
        self.vs = np.zeros((B, H, cap, D // G), md)
        self.vz = np.zeros((B, H, cap, D // G), md)
        self.k_res = np.zeros((B, H, R, D), np.uint16)
        self.v_res = np.zeros((B, H, R, D), np.uint16)
        self.k_outl = (np.zeros(outlier_shape(B, H, cap, G, self.n_out, D), np.uint32)
                       if self.n_out else None)

    def prefill(self, k, v, tq):
        """Quantize tokens [0, tq) and keep tokens [tq, T) in the residual."""
        k, v = _h(k), _h(v)
        T = k.shape[2]
        if not (0 <= T - tq <= self.R):
            raise OracleError("ESHAPE")
        if tq:
            quantize_k(k, self.bits, self.G, self.cap, tq, 0, self.k_codes, self.ks, self.kz,
                       self.meta_half, self.n_out, self.k_outl)
        self.k_res[:, :, : T - tq] = k[:, :, tq:]
        if self.v_window:
            # values [0, T - R) quantized one token at a time, the rest in the
            # window at slot t % R
            tv = max(0, T - self.R)
            for t in range(tv):
                quantize_v_token(v, t, t, self.bits, self.G, self.cap, self.v_codes, self.vs,
                                 self.vz, self.meta_half)
            for t in range(tv, T):
                self.v_res[:, :, t % self.R] = v[:, :, t]
        else:
            if tq:
                quantize_v(v, self.bits, self.G, self.cap, tq, 0, self.v_codes, self.vs,
                           self.vz, self.meta_half)
            self.v_res[:, :, : T - tq] = v[:, :, tq:]
        self.tq, self.tr = tq, T - tq

    def append(self, k_new, v_new):
        k_new, v_new = _h(k_new), _h(v_new)
        tq = ctypes.c_int(self.tq)
        tr = ctypes.c_int(self.tr)
        before = self.tq
        mh = self.meta_half
        fn = load().kivio_append_vw if self.v_window else load().kivio_append
        _check(fn(
            self.B, self.H, self.D, self.bits, self.G, self.R, self.cap, int(mh),
            _p(self.k_codes, ctypes.c_uint32, np.uint32), _m(self.ks, mh), _m(self.kz, mh),
            _p(self.v_codes, ctypes.c_uint32, np.uint32), _m(self.vs, mh), _m(self.vz, mh),
            _p(self.k_res, ctypes.c_uint16, np.uint16), _p(self.v_res, ctypes.c_uint16, np.uint16),
            _p(k_new, ctypes.c_uint16, np.uint16), _p(v_new, ctypes.c_uint16, np.uint16),
            ctypes.byref(tq), ctypes.byref(tr), int(self.n_out), _outl(self.k_outl)))
        self.tq, self.tr = tq.value, tr.value
        if self.tq != before:
            self.flushes += 1

    @property
    def tv(self) -> int:
        """Quantized value tokens (tq without the value window)."""
        return max(0, self.tq + self.tr - self.R) if self.v_window else self.tq

    def decode(self, q, softmax_scale):
        return decode_attn(self, q, softmax_scale)


def decode_attn(c: OracleCache, q, softmax_scale):
    """Binary64 attention output [B][H*r][D] for decode queries q (binary16)."""
    q = _h(q)
    assert q.shape == (c.B, c.H * c.r, c.D), q.shape
    out = np.zeros((c.B, c.H * c.r, c.D), np.float64)
    scratch = np.zeros(2 * max(1, c.tq + c.tr), np.float64)
    mh = c.meta_half
    _check(load().kivio_decode_attn_vw(
        c.B, c.H, c.r, c.D, c.bits, c.G, c.R, c.cap, int(mh),
        _p(c.k_codes, ctypes.c_uint32, np.uint32), _m(c.ks, mh), _m(c.kz, mh),
        _p(c.v_codes, ctypes.c_uint32, np.uint32), _m(c.vs, mh), _m(c.vz, mh),
        _p(c.k_res, ctypes.c_uint16, np.uint16), _p(c.v_res, ctypes.c_uint16, np.uint16),
        c.tq, c.tr, _p(q, ctypes.c_uint16, np.uint16), float(softmax_scale),
        _p(out, ctypes.c_double, np.float64), _p(scratch, ctypes.c_double, np.float64),
        int(c.n_out), _outl(c.k_outl), float(c.rope_theta), int(c.v_window)))
    return out

"""C ABI checks that need no GPU: the library loads, exports every symbol
include/kivi.h declares, and rejects bad arguments before any HIP call
(nothing is enqueued and the cache lengths stay unchanged)."""
import ctypes
import os
import re

import pytest

from kv_cache_bit_kivi_amd import _lib
from kv_cache_bit_kivi_amd._lib import (KIVI_EALIGN, KIVI_ECAPACITY, KIVI_EINVAL, KIVI_ESHAPE,
                                        KIVI_EUNSUPPORTED, KIVI_EWORKSPACE, KIVI_OK, kivi_cache,
                                        kivi_shape)

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "kivi.h")
P = 4096  # fake 16-byte aligned "device" address: never dereferenced on error paths


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kivi_\w+)\s*\(", text)))


def test_exports_match_header():
    names = declared()
    assert len(names) >= 9
    L = _lib.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(_lib.PROTOTYPES) == names


def test_strerror():
    for code in range(8):
        assert _lib.kivi_strerror(code)
    assert _lib.kivi_strerror(99) == b"unknown status"


def shape(**kw):
    d = dict(batch=2, num_kv_heads=4, gqa_ratio=2, head_dim=128, bits=2, group=32,
             residual=128, capacity=512, meta_half=0, outliers=0, rope_theta=0.0,
             deterministic=0, v_window=0)
    d.update(kw)
    return kivi_shape(*[d[n] for n, _ in kivi_shape._fields_])


def sizes(s):
    out = [ctypes.c_size_t() for _ in range(6)]
    rc = _lib.kivi_cache_bytes(ctypes.byref(s), *[ctypes.byref(x) for x in out])
    return rc, [x.value for x in out]


def test_cache_bytes():
    rc, sz = sizes(shape())
    assert rc == KIVI_OK
    planes, cap, D = 8, 512, 128
    assert sz == [planes * cap * D // 4, planes * cap // 32 * D * 4, planes * cap * D // 4,
                  planes * cap * 4 * 4, planes * 128 * D * 2, planes * 2 * D * 2]
    rc, sz = sizes(shape(bits=4))
    assert sz[0] == planes * cap * D // 2
    for b in (1, 3):      # one- and three-bit codes: D*b/32 words per key row
        rc, sz = sizes(shape(bits=b))
        assert rc == KIVI_OK and sz[0] == sz[2] == planes * cap * D * b // 8
    # binary16 metadata: half the scale / zero bytes, nothing else changes
    rc, sz16 = sizes(shape(meta_half=1))
    assert rc == KIVI_OK
    _, sz32 = sizes(shape())
    assert sz16[1] * 2 == sz32[1] and sz16[3] * 2 == sz32[3]
    assert [sz16[i] for i in (0, 2, 4, 5)] == [sz32[i] for i in (0, 2, 4, 5)]


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), KIVI_EINVAL), (dict(num_kv_heads=0), KIVI_EINVAL),
    (dict(gqa_ratio=0), KIVI_EINVAL), (dict(bits=0), KIVI_EINVAL), (dict(bits=5), KIVI_EINVAL),
    (dict(bits=8), KIVI_EINVAL),
    (dict(head_dim=48), KIVI_EUNSUPPORTED), (dict(group=16), KIVI_EUNSUPPORTED),
    (dict(gqa_ratio=17), KIVI_EUNSUPPORTED), (dict(head_dim=32, group=64), KIVI_ESHAPE),
    (dict(residual=48), KIVI_ESHAPE), (dict(residual=16, group=32), KIVI_ESHAPE),
    (dict(capacity=96), KIVI_ESHAPE), (dict(capacity=-64), KIVI_ESHAPE),
    (dict(group=128, capacity=192), KIVI_ESHAPE),
    (dict(meta_half=2), KIVI_EINVAL), (dict(meta_half=-1), KIVI_EINVAL),
    (dict(outliers=-1), KIVI_EINVAL), (dict(outliers=9), KIVI_EINVAL),
    (dict(rope_theta=-1.0), KIVI_EINVAL), (dict(rope_theta=float("inf")), KIVI_EINVAL),
    (dict(rope_theta=float("nan")), KIVI_EINVAL),
    (dict(deterministic=2), KIVI_EINVAL), (dict(deterministic=-1), KIVI_EINVAL),
    (dict(v_window=2), KIVI_EINVAL), (dict(v_window=-1), KIVI_EINVAL),
])
def test_shape_errors(kw, code):
    assert sizes(shape(**kw))[0] == code


def qk(s, x=P, stride=256, ntok=64, dst=0, codes=P, sc=P, zr=P):
    return _lib.kivi_quantize_k(ctypes.byref(s), x, stride, ntok, dst, codes, sc, zr, None)


def qv(s, x=P, stride=256, ntok=64, dst=0, codes=P, sc=P, zr=P):
    return _lib.kivi_quantize_v(ctypes.byref(s), x, stride, ntok, dst, codes, sc, zr, None)


@pytest.mark.parametrize("fn", [qk, qv])
def test_quantize_errors(fn):
    s = shape()
    assert fn(s, x=None) == KIVI_EINVAL
    assert fn(s, codes=None) == KIVI_EINVAL
    assert fn(s, x=P + 2) == KIVI_EALIGN
    assert fn(s, zr=P + 8) == KIVI_EALIGN
    assert fn(s, ntok=0) == KIVI_ESHAPE
    assert fn(s, ntok=48) == KIVI_ESHAPE
    assert fn(s, dst=16) == KIVI_ESHAPE
    assert fn(s, dst=-32) == KIVI_ESHAPE
    assert fn(s, stride=32, ntok=64) == KIVI_ESHAPE
    assert fn(s, ntok=64, dst=480) == KIVI_ECAPACITY
    assert fn(shape(bits=5)) == KIVI_EINVAL


def cache(**kw):
    tq = kw.pop("tq", 0)
    tr = kw.pop("tr", 0)
    ptrs = kw.pop("ptrs", [P] * 8)
    k_out = kw.pop("k_out", None)
    return kivi_cache(shape(**kw), *ptrs, tq, tr, k_out)


# ---- key outliers ----

def test_outlier_bytes():
    n = ctypes.c_size_t()
    s = shape(outliers=2)
    assert _lib.kivi_outlier_bytes(ctypes.byref(s), 0, 0, ctypes.byref(n)) == KIVI_OK
    assert n.value == 8 * (512 // 32) * 2 * 128 * 4           # planes x groups x n x D words
    assert _lib.kivi_outlier_bytes(ctypes.byref(s), 256, 10, ctypes.byref(n)) == KIVI_OK
    assert n.value == 10 * 4 * (256 // 32) * 2 * 128 * 4      # pages x heads x ...
    assert _lib.kivi_outlier_bytes(ctypes.byref(shape()), 0, 0, ctypes.byref(n)) == KIVI_OK
    assert n.value == 0
    assert _lib.kivi_outlier_bytes(ctypes.byref(s), 96, 10, ctypes.byref(n)) == KIVI_ESHAPE
    assert _lib.kivi_outlier_bytes(ctypes.byref(s), 0, 0, None) == KIVI_EINVAL
    assert _lib.kivi_outlier_bytes(ctypes.byref(shape(outliers=9)), 0, 0,
                                   ctypes.byref(n)) == KIVI_EINVAL


def test_quantize_outlier_errors():
    qo = _lib.kivi_quantize_k_outliers
    s = shape(outliers=1)
    assert qk(s) == KIVI_EINVAL                     # plain call on an outlier shape
    assert qo(ctypes.byref(s), P, 256, 64, 0, P, P, P, None, None) == KIVI_EINVAL
    assert qo(ctypes.byref(s), P, 256, 64, 0, P, P, P, P + 4, None) == KIVI_EALIGN
    assert qo(ctypes.byref(shape()), P, 256, 64, 0, P, P, P, P, None) == KIVI_EINVAL
    assert qo(ctypes.byref(s), P, 256, 48, 0, P, P, P, P, None) == KIVI_ESHAPE
    assert qo(ctypes.byref(s), P, 256, 64, 480, P, P, P, P, None) == KIVI_ECAPACITY


def test_outlier_cache_needs_its_store():
    import numpy as np
    c = cache(outliers=1, tq=64, tr=3)
    assert _lib.kivi_append(ctypes.byref(c), P, P, None) == KIVI_EINVAL
    assert _lib.kivi_decode_attn(ctypes.byref(c), P, 0.1, P, None, 0, 1, None) == KIVI_EINVAL
    assert _lib.kivi_prefill(ctypes.byref(c), P, P, 64, 64, None) == KIVI_EINVAL
    assert (c.tq, c.tr) == (64, 3)
    c = cache(outliers=1, tq=64, tr=3, k_out=P + 8)
    assert _lib.kivi_append(ctypes.byref(c), P, P, None) == KIVI_EALIGN
    r = ragged([64, 32], [3, 1], outliers=2)
    assert _lib.kivi_ragged_append(ctypes.byref(r), P, P, None) == KIVI_EINVAL
    assert lens(r) == ([64, 32], [3, 1])
    g = paged([64, 32], [3, 1], outliers=2)
    assert _lib.kivi_paged_decode_attn(ctypes.byref(g), P, 0.1, P, None, 0, 1, None) == KIVI_EINVAL
    assert np.array_equal(g._keep[0], [64, 32])


def test_append_errors_leave_state():
    c = cache(tq=416, tr=128)          # the flush would end at 544 > capacity 512
    assert _lib.kivi_append(ctypes.byref(c), P, P, None) == KIVI_ECAPACITY
    assert (c.tq, c.tr) == (416, 128)
    c = cache(tq=32 + 1, tr=0)
    assert _lib.kivi_append(ctypes.byref(c), P, P, None) == KIVI_ESHAPE
    c = cache(tq=0, tr=129)
    assert _lib.kivi_append(ctypes.byref(c), P, P, None) == KIVI_ESHAPE
    assert (c.tq, c.tr) == (0, 129)
    c = cache()
    assert _lib.kivi_append(ctypes.byref(c), None, P, None) == KIVI_EINVAL
    assert _lib.kivi_append(ctypes.byref(c), P + 4, P, None) == KIVI_EALIGN
    c = cache(ptrs=[P] * 7 + [0])
    assert _lib.kivi_append(ctypes.byref(c), P, P, None) == KIVI_EINVAL
    c = cache(ptrs=[P] * 3 + [P + 8] + [P] * 4)
    assert _lib.kivi_append(ctypes.byref(c), P, P, None) == KIVI_EALIGN
    c = cache(tq=1024, tr=0)
    assert _lib.kivi_append(ctypes.byref(c), P, P, None) == KIVI_ECAPACITY
    assert (c.tq, c.tr) == (1024, 0)


def test_prefill_errors():
    c = cache()
    assert _lib.kivi_prefill(ctypes.byref(c), P, P, 300, 128, None) == KIVI_ESHAPE  # tr > R
    assert _lib.kivi_prefill(ctypes.byref(c), P, P, 100, 48, None) == KIVI_ESHAPE   # tq % G
    assert _lib.kivi_prefill(ctypes.byref(c), P, P, 0, 0, None) == KIVI_ESHAPE
    assert _lib.kivi_prefill(ctypes.byref(c), P, P, 600, 544, None) == KIVI_ECAPACITY
    assert _lib.kivi_prefill(ctypes.byref(c), None, P, 64, 64, None) == KIVI_EINVAL
    assert (c.tq, c.tr) == (0, 0)


def test_decode_errors():
    c = cache(tq=0, tr=0)
    dec = _lib.kivi_decode_attn
    assert dec(ctypes.byref(c), P, 0.1, P, None, 0, 1, None) == KIVI_ESHAPE   # empty cache
    c = cache(tq=64, tr=3)
    assert dec(ctypes.byref(c), None, 0.1, P, None, 0, 1, None) == KIVI_EINVAL
    assert dec(ctypes.byref(c), P, 0.1, P + 2, None, 0, 1, None) == KIVI_EALIGN
    assert dec(ctypes.byref(c), P, 0.1, P, None, 0, -1, None) == KIVI_EINVAL
    assert dec(ctypes.byref(c), P, 0.1, P, None, 0, 68, None) == KIVI_ESHAPE  # splits > tokens
    need = _lib.kivi_decode_workspace_bytes(ctypes.byref(c.shape), 4)
    assert dec(ctypes.byref(c), P, 0.1, P, P, need - 1, 4, None) == KIVI_EWORKSPACE
    assert dec(ctypes.byref(c), P, 0.1, P, None, need, 4, None) == KIVI_EINVAL
    assert dec(ctypes.byref(c), P, 0.1, P, P + 4, need, 4, None) == KIVI_EALIGN
    c = cache(tq=64, tr=200)
    assert dec(ctypes.byref(c), P, 0.1, P, None, 0, 1, None) == KIVI_ESHAPE
    # at most KIVI_MAX_SPLITS = 4096 splits, even with more tokens than that
    c = cache(tq=4224, tr=100, capacity=4352)
    need = _lib.kivi_decode_workspace_bytes(ctypes.byref(c.shape), 4096)
    assert need > 0 and _lib.kivi_decode_workspace_bytes(ctypes.byref(c.shape), 4097) == 0
    assert dec(ctypes.byref(c), P, 0.1, P, P, 1 << 40, 4097, None) == KIVI_ESHAPE


def test_workspace_bytes():
    s = shape()
    ws = _lib.kivi_decode_workspace_bytes
    assert ws(ctypes.byref(s), 1) == 0
    rows = 2 * 4 * 2
    assert ws(ctypes.byref(s), 4) == rows * 4 * (128 + 2) * 4
    assert ws(ctypes.byref(s), 0) >= ws(ctypes.byref(s), 4)
    assert ws(ctypes.byref(shape(bits=5)), 4) == 0


def test_append_decode_errors_leave_state():
    """The fused step checks the append's and the (post-append) decode's
    conditions before enqueueing anything."""
    ad = _lib.kivi_append_decode_attn
    c = cache(tq=416, tr=128)          # the flush would end at 544 > capacity 512
    assert ad(ctypes.byref(c), P, P, P, 0.1, P, None, 0, 1, None) == KIVI_ECAPACITY
    assert (c.tq, c.tr) == (416, 128)
    c = cache(tq=64, tr=3)
    assert ad(ctypes.byref(c), None, P, P, 0.1, P, None, 0, 1, None) == KIVI_EINVAL
    assert ad(ctypes.byref(c), P, P + 4, P, 0.1, P, None, 0, 1, None) == KIVI_EALIGN
    assert ad(ctypes.byref(c), P, P, None, 0.1, P, None, 0, 1, None) == KIVI_EINVAL
    assert ad(ctypes.byref(c), P, P, P, 0.1, P + 2, None, 0, 1, None) == KIVI_EALIGN
    assert ad(ctypes.byref(c), P, P, P, 0.1, P, None, 0, -1, None) == KIVI_EINVAL
    # 64 + 4 tokens after the append: 68 splits are allowed, 69 are not
    assert ad(ctypes.byref(c), P, P, P, 0.1, P, None, 0, 69, None) == KIVI_ESHAPE
    need = _lib.kivi_decode_workspace_bytes(ctypes.byref(c.shape), 4)
    assert ad(ctypes.byref(c), P, P, P, 0.1, P, P, need - 1, 4, None) == KIVI_EWORKSPACE
    assert ad(ctypes.byref(c), P, P, P, 0.1, P, None, need, 4, None) == KIVI_EINVAL
    assert (c.tq, c.tr) == (64, 3)
    c = cache(ptrs=[P] * 7 + [0])
    assert ad(ctypes.byref(c), P, P, P, 0.1, P, None, 0, 1, None) == KIVI_EINVAL


# ---- ragged batches: validation before any HIP call, lengths untouched ----

def ragged(tq, tr, ptrs=None, **kw):
    """A ragged cache over fake device pointers; tq / tr are kept alive on the
    returned struct (the C side reads and writes them in place)."""
    import numpy as np
    from kv_cache_bit_kivi_amd._lib import kivi_ragged_cache
    s = shape(**kw)
    tqa = np.ascontiguousarray(tq, np.int32)
    tra = np.ascontiguousarray(tr, np.int32)
    assert len(tqa) == s.batch and len(tra) == s.batch
    p32 = ctypes.POINTER(ctypes.c_int32)
    c = kivi_ragged_cache(s, *(ptrs or [P] * 8), tqa.ctypes.data_as(p32),
                          tra.ctypes.data_as(p32), None)
    c._keep = (tqa, tra)
    return c


def lens(c):
    return c._keep[0].tolist(), c._keep[1].tolist()


def test_ragged_append_errors_leave_state():
    ap = _lib.kivi_ragged_append
    c = ragged([416, 0], [128, 5])       # sequence 0 would flush past capacity 512
    assert ap(ctypes.byref(c), P, P, None) == KIVI_ECAPACITY
    assert lens(c) == ([416, 0], [128, 5])
    c = ragged([64, 33], [1, 1])         # tq not a multiple of the group
    assert ap(ctypes.byref(c), P, P, None) == KIVI_ESHAPE
    c = ragged([64, 32], [1, 129])       # residual longer than R
    assert ap(ctypes.byref(c), P, P, None) == KIVI_ESHAPE
    assert lens(c) == ([64, 32], [1, 129])
    c = ragged([64, 1024], [1, 0])       # past capacity
    assert ap(ctypes.byref(c), P, P, None) == KIVI_ECAPACITY
    c = ragged([0, 0], [0, 0])
    assert ap(ctypes.byref(c), None, P, None) == KIVI_EINVAL
    assert ap(ctypes.byref(c), P, P + 4, None) == KIVI_EALIGN
    c = ragged([0, 0], [0, 0], ptrs=[P] * 7 + [0])
    assert ap(ctypes.byref(c), P, P, None) == KIVI_EINVAL
    c = ragged([0, 0], [0, 0])
    c.tq = None
    assert ap(ctypes.byref(c), P, P, None) == KIVI_EINVAL


def test_ragged_prefill_errors():
    import numpy as np
    pf = _lib.kivi_ragged_prefill
    p32 = ctypes.POINTER(ctypes.c_int32)

    def call(c, stride, ntok, tq, k=P):
        n = np.asarray(ntok, np.int32)
        t = np.asarray(tq, np.int32)
        return pf(ctypes.byref(c), k, P, stride, n.ctypes.data_as(p32), t.ctypes.data_as(p32),
                  None)

    c = ragged([0, 0], [0, 0])
    assert call(c, 256, [300, 64], [256, 64]) == KIVI_ESHAPE    # ntok > stride
    assert call(c, 512, [300, 64], [128, 64]) == KIVI_ESHAPE    # residual part > R
    assert call(c, 256, [100, 64], [48, 64]) == KIVI_ESHAPE     # tq % G
    assert call(c, 256, [10, 64], [32, 64]) == KIVI_ESHAPE      # tq > ntok
    assert call(c, 640, [600, 64], [544, 64]) == KIVI_ECAPACITY
    assert call(c, 0, [0, 0], [0, 0]) == KIVI_ESHAPE            # stride < 1
    assert call(c, 64, [64, 64], [64, 64], k=None) == KIVI_EINVAL
    assert call(c, 64, [64, 64], [64, 64], k=P + 2) == KIVI_EALIGN
    assert lens(c) == ([0, 0], [0, 0])


def test_ragged_decode_errors():
    dec = _lib.kivi_ragged_decode_attn
    c = ragged([64, 0], [3, 0])          # sequence 1 is empty
    assert dec(ctypes.byref(c), P, 0.1, P, None, 0, 1, None) == KIVI_ESHAPE
    c = ragged([64, 32], [3, 1])
    assert dec(ctypes.byref(c), None, 0.1, P, None, 0, 1, None) == KIVI_EINVAL
    assert dec(ctypes.byref(c), P, 0.1, P + 2, None, 0, 1, None) == KIVI_EALIGN
    assert dec(ctypes.byref(c), P, 0.1, P, None, 0, -1, None) == KIVI_EINVAL
    need = _lib.kivi_decode_workspace_bytes(ctypes.byref(c.shape), 4)
    assert dec(ctypes.byref(c), P, 0.1, P, P, need - 1, 4, None) == KIVI_EWORKSPACE
    assert dec(ctypes.byref(c), P, 0.1, P, None, need, 4, None) == KIVI_EINVAL
    assert dec(ctypes.byref(c), P, 0.1, P, P + 4, need, 4, None) == KIVI_EALIGN
    c = ragged([64, 32], [3, 200])
    assert dec(ctypes.byref(c), P, 0.1, P, None, 0, 1, None) == KIVI_ESHAPE


def test_ragged_append_decode_errors_leave_state():
    ad = _lib.kivi_ragged_append_decode_attn
    c = ragged([416, 64], [128, 7])      # sequence 0's flush would pass capacity
    assert ad(ctypes.byref(c), P, P, P, 0.1, P, None, 0, 1, None) == KIVI_ECAPACITY
    assert lens(c) == ([416, 64], [128, 7])
    c = ragged([0, 0], [0, 0])           # empty before, one token each after: valid sizes
    assert ad(ctypes.byref(c), P, P, None, 0.1, P, None, 0, 1, None) == KIVI_EINVAL
    assert ad(ctypes.byref(c), P, P, P, 0.1, P, None, 0, -1, None) == KIVI_EINVAL
    need = _lib.kivi_decode_workspace_bytes(ctypes.byref(c.shape), 4)
    assert ad(ctypes.byref(c), P, P, P, 0.1, P, P, need - 1, 4, None) == KIVI_EWORKSPACE
    assert lens(c) == ([0, 0], [0, 0])


# ---- paged store: page-size / pool validation, then the ragged rules ----

def paged(tq, tr, page_tokens=128, num_pages=16, table=P, ptrs=None, **kw):
    import numpy as np
    from kv_cache_bit_kivi_amd._lib import kivi_paged_cache
    s = shape(**kw)
    tqa = np.ascontiguousarray(tq, np.int32)
    tra = np.ascontiguousarray(tr, np.int32)
    p32 = ctypes.POINTER(ctypes.c_int32)
    c = kivi_paged_cache(s, page_tokens, num_pages, *(ptrs or [P] * 8), table,
                         tqa.ctypes.data_as(p32), tra.ctypes.data_as(p32), None)
    c._keep = (tqa, tra)
    return c


def test_paged_pool_bytes():
    out = [ctypes.c_size_t() for _ in range(4)]
    s = shape(meta_half=1)
    assert _lib.kivi_paged_pool_bytes(ctypes.byref(s), 256, 10, *[ctypes.byref(x) for x in out]) == 0
    slices = 10 * 4
    assert [x.value for x in out] == [slices * 256 * 128 // 4, slices * 8 * 128 * 2,
                                      slices * 256 * 128 // 4, slices * 256 * 4 * 2]
    bad = [(96, 10), (32, 10), (192, 10), (128, 0)]     # not a power of two, < 64, ..., no pages
    for pt, npg in bad:
        assert _lib.kivi_paged_pool_bytes(ctypes.byref(s), pt, npg, None, None, None,
                                          None) == KIVI_ESHAPE
    s = shape(group=128)
    assert _lib.kivi_paged_pool_bytes(ctypes.byref(s), 64, 4, None, None, None, None) == KIVI_ESHAPE


def test_paged_errors_leave_state():
    ad = _lib.kivi_paged_append_decode_attn
    ap = _lib.kivi_paged_append
    dec = _lib.kivi_paged_decode_attn
    c = paged([416, 64], [128, 7])       # sequence 0's flush would pass capacity 512
    assert ap(ctypes.byref(c), P, P, None) == KIVI_ECAPACITY
    assert ad(ctypes.byref(c), P, P, P, 0.1, P, None, 0, 1, None) == KIVI_ECAPACITY
    assert lens(c) == ([416, 64], [128, 7])
    c = paged([64, 32], [3, 1], page_tokens=96)          # page size not a power of two
    assert dec(ctypes.byref(c), P, 0.1, P, None, 0, 1, None) == KIVI_ESHAPE
    c = paged([64, 32], [3, 1], page_tokens=1024)        # capacity 512 not a multiple
    assert dec(ctypes.byref(c), P, 0.1, P, None, 0, 1, None) == KIVI_ESHAPE
    c = paged([64, 32], [3, 1], num_pages=0)
    assert dec(ctypes.byref(c), P, 0.1, P, None, 0, 1, None) == KIVI_ESHAPE
    c = paged([64, 32], [3, 1], table=None)
    assert dec(ctypes.byref(c), P, 0.1, P, None, 0, 1, None) == KIVI_EINVAL
    c = paged([64, 32], [3, 1], table=P + 2)             # block table not 4-byte aligned
    assert dec(ctypes.byref(c), P, 0.1, P, None, 0, 1, None) == KIVI_EALIGN
    c = paged([64, 0], [3, 0])                           # sequence 1 empty
    assert dec(ctypes.byref(c), P, 0.1, P, None, 0, 1, None) == KIVI_ESHAPE
    c = paged([64, 32], [3, 1], ptrs=[P] * 7 + [0])
    assert ap(ctypes.byref(c), P, P, None) == KIVI_EINVAL
    assert lens(c) == ([64, 32], [3, 1])


def test_one_hip_runtime_in_process():
    """Loading the library first (before torch) must not map a second HIP
    runtime next to PyTorch's: a fresh interpreter loads it through the
    binding, then imports torch, and exactly one libamdhip64 is mapped."""
    import subprocess
    import sys
    code = ("from kv_cache_bit_kivi_amd import _lib; _lib.lib(); import torch; "
            "paths = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}; "
            "print(len(paths), sorted(paths))")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                         timeout=600)
    assert out.returncode == 0, out.stderr
    n = int(out.stdout.split()[0])
    assert n == 1, out.stdout


# ---- value window ----

def test_window_errors_leave_state():
    """The window append and the fused step refuse a key flush or a value
    past the capacity, and bad arguments, before any HIP call; ragged and
    paged caches refuse the window."""
    import numpy as np
    ad = _lib.kivi_append_decode_attn
    c = cache(tq=416, tr=128, v_window=1)      # key flush to 544 > 512
    assert _lib.kivi_append(ctypes.byref(c), P, P, None) == KIVI_ECAPACITY
    assert ad(ctypes.byref(c), P, P, P, 0.1, P, None, 0, 1, None) == KIVI_ECAPACITY
    assert (c.tq, c.tr) == (416, 128)
    c = cache(tq=64, tr=3, v_window=1)
    assert _lib.kivi_append(ctypes.byref(c), None, P, None) == KIVI_EINVAL
    assert ad(ctypes.byref(c), P, P, P, 0.1, P + 2, None, 0, 1, None) == KIVI_EALIGN
    # the query covers the window's extra partial slot (its tail) ...
    ws = _lib.kivi_decode_workspace_bytes
    assert ws(ctypes.byref(c.shape), 4) == ws(ctypes.byref(shape()), 5)
    # (automatic: at most 2048 / 8 = 256 splits for 2 x 4 (b, h) units, + 1)
    assert ws(ctypes.byref(c.shape), 0) == ws(ctypes.byref(shape()), 0) // 256 * 257
    # ... and a workspace short of this decode's own 4 slots is refused
    need = ws(ctypes.byref(shape()), 4)
    assert ad(ctypes.byref(c), P, P, P, 0.1, P, P, need - 1, 4, None) == KIVI_EWORKSPACE
    assert (c.tq, c.tr) == (64, 3)
    assert _lib.kivi_prefill(ctypes.byref(c), P, P, 300, 128, None) == KIVI_ESHAPE
    assert (c.tq, c.tr) == (64, 3)
    r = ragged([64, 32], [3, 1], v_window=1)
    assert _lib.kivi_ragged_append(ctypes.byref(r), P, P, None) == KIVI_EUNSUPPORTED
    p32 = ctypes.POINTER(ctypes.c_int32)
    assert _lib.kivi_ragged_prefill(ctypes.byref(r), P, P, 256, r._keep[0].ctypes.data_as(p32),
                                    r._keep[1].ctypes.data_as(p32), None) == KIVI_EUNSUPPORTED
    assert lens(r) == ([64, 32], [3, 1])
    g = paged([64, 32], [3, 1], v_window=1)
    assert _lib.kivi_paged_decode_attn(ctypes.byref(g), P, 0.1, P, None, 0, 1,
                                       None) == KIVI_EUNSUPPORTED
    assert np.array_equal(g._keep[0], [64, 32])

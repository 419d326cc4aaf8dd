"""kivi_decode_attn_noalloc: the decode whose split-K partials live in the
library's own device array (for callers that cannot allocate).  Argument
checks run on the CPU; on the GPU its output equals kivi_decode_attn's with a
caller workspace, bit for bit (deterministic caches, the same split count),
over two calls in a row, the second one smaller, on both kernel paths."""
import ctypes

import numpy as np
import pytest

from kv_cache_bit_kivi_amd import _lib
from kv_cache_bit_kivi_amd._lib import (KIVI_EALIGN, KIVI_EINVAL, KIVI_ESHAPE, KIVI_EWORKSPACE,
                                        kivi_cache, kivi_shape)

P = 4096  # fake aligned address: never dereferenced on the error paths
SCRATCH = 8 << 20


def _cache(batch=2, heads=4, r=2, D=128, tq=64, tr=3, cap=1024):
    s = kivi_shape(batch, heads, r, D, 2, 32, 32, cap, 0, 0, 0.0, 1)
    return kivi_cache(s, P, P, P, P, P, P, P, P, tq, tr, None)


def test_noalloc_rejects_before_any_hip_call():
    fn = _lib.kivi_decode_attn_noalloc
    c = _cache(tq=0, tr=0)
    assert fn(ctypes.byref(c), P, 0.1, P, 1, None) == KIVI_ESHAPE       # empty cache
    c = _cache()
    assert fn(ctypes.byref(c), None, 0.1, P, 1, None) == KIVI_EINVAL
    assert fn(ctypes.byref(c), P, 0.1, P + 2, 1, None) == KIVI_EALIGN
    assert fn(ctypes.byref(c), P, 0.1, P, -1, None) == KIVI_EINVAL
    assert fn(ctypes.byref(c), P, 0.1, P, 68, None) == KIVI_ESHAPE      # splits > tokens
    # partials larger than the array: 64 x 32 rows x 16 splits x 130 floats
    c = _cache(batch=64, heads=32, r=1, tq=4096, tr=5, cap=4224)
    need = _lib.kivi_decode_workspace_bytes(ctypes.byref(c.shape), 16)
    assert need > SCRATCH
    assert fn(ctypes.byref(c), P, 0.1, P, 16, None) == KIVI_EWORKSPACE
    ok = max(s for s in range(1, 17)
             if _lib.kivi_decode_workspace_bytes(ctypes.byref(c.shape), s) <= SCRATCH)
    assert ok >= 7
    assert fn(ctypes.byref(c), P, 0.1, P, ok + 1, None) == KIVI_EWORKSPACE


@pytest.mark.gpu
def test_noalloc_equals_workspace_decode():
    import torch

    from kv_cache_bit_kivi_amd import synth
    from kv_cache_bit_kivi_amd.cache import KiviCache
    from tests.gpu_util import announce, dev, host, require_gpu

    require_gpu()
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    # (B, H, r, D, bits, G, R, tq, tr, splits, value window): a long matrix-core
    # case, then a smaller one; a generic-kernel case (D = 64); the automatic
    # split count; value windows (matrix cores + the tail kernel, whose
    # partials go through the array; the generic kernel alone)
    cases = [(4, 8, 2, 128, 2, 32, 128, 2944, 77, 5, False),
             (2, 4, 1, 128, 4, 32, 64, 640, 9, 3, False),
             (3, 2, 1, 64, 2, 32, 32, 448, 20, 4, False),
             (1, 2, 1, 128, 2, 32, 128, 16256, 100, 0, False),
             (2, 4, 2, 128, 2, 32, 128, 960, 100, 3, True),
             (2, 4, 2, 64, 2, 32, 64, 256, 40, 0, True)]
    for i, (B, H, r, D, bits, G, R, tq, tr, S, vw) in enumerate(cases):
        announce(f"noalloc vs workspace decode {(B, H, r, D, bits, G, R, tq, tr, S, vw)}")
        T = tq + tr
        cap = (T + 63) // 64 * 64
        k = synth.random_fp16(500 + i, (B, H, T, D), scale=2.0)
        v = synth.random_fp16(600 + i, (B, H, T, D))
        q = dev(synth.random_fp16(700 + i, (B, H * r, D)))
        gc = KiviCache(B, H, r, D, bits, G, R, cap, deterministic=True, v_window=vw)
        gc.prefill(dev(k), dev(v), tq)
        splits = S if S else gc.auto_splits()
        if S == 0:
            assert splits > 1
        ws = gc.workspace_for(splits)
        ref = torch.empty_like(q)
        got = torch.full_like(q, float("nan"))
        rc = _lib.kivi_decode_attn(ctypes.byref(gc.c), q.data_ptr(), 0.08, ref.data_ptr(),
                                   None if ws is None else ws.data_ptr(),
                                   0 if ws is None else ws.numel(), S, stream)
        assert rc == 0, rc
        rc = _lib.kivi_decode_attn_noalloc(ctypes.byref(gc.c), q.data_ptr(), 0.08,
                                           got.data_ptr(), S, stream)
        assert rc == 0, rc
        a, b = host(ref).view(np.uint16), host(got).view(np.uint16)
        assert np.array_equal(a, b), (i, int(np.sum(a != b)))

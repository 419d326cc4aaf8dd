"""Helpers for the GPU parity tests (marked `gpu`).

Inputs come from kv_cache_bit_kivi_amd.synth (seeded, shared by both sides);
expected values come from the C oracle only.  When a GPU is present but the
HIP library is missing, the tests fail (no fallback path exists)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_bit_kivi_amd import _lib
    _lib.lib()  # raises ImportError when libkivi.so is missing


def announce(msg: str) -> None:
    """Name the case on stdout before its GPU work starts."""
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.float16:
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    a = t.cpu().numpy()
    if a.dtype == np.int32:
        a = a.view(np.uint32)
    return a


def gpu_cache_from_oracle_shape(oc, device="cuda"):
    from kv_cache_bit_kivi_amd.cache import KiviCache
    return KiviCache(oc.B, oc.H, oc.r, oc.D, oc.bits, oc.G, oc.R, oc.cap, device=device,
                     meta_half=oc.meta_half, outliers=oc.n_out)


def assert_cache_equal(gc, oc, planes=None, what=""):
    """Bit-exact comparison of every cache buffer (optionally a batch subset:
    ``planes`` lists the batch indices of the GPU cache that the oracle cache's
    batch entries correspond to)."""
    assert (gc.tq, gc.tr) == (oc.tq, oc.tr), what
    pairs = [("k_codes", "k_codes"), ("k_scale", "ks"), ("k_zero", "kz"),
             ("v_codes", "v_codes"), ("v_scale", "vs"), ("v_zero", "vz")]
    for gname, oname in pairs:
        g = getattr(gc, gname)
        if planes is not None:
            g = g[list(planes)]
        g = host(g)
        o = getattr(oc, oname)
        if g.dtype == np.float32:
            g, o = g.view(np.uint32), o.view(np.uint32)
        elif g.dtype == np.float16:           # binary16 metadata: compare the bits
            g = g.view(np.uint16)
            assert o.dtype == np.uint16, (gname, o.dtype)
        if not np.array_equal(g, o):
            bad = np.argwhere(g != o)
            raise AssertionError(f"{what} {gname}: {len(bad)} mismatches, first at "
                                 f"{bad[0].tolist()}: gpu={g[tuple(bad[0])]} oracle={o[tuple(bad[0])]}")
    if oc.n_out:
        g = gc.k_outliers
        if planes is not None:
            g = g[list(planes)]
        g = host(g)
        if not np.array_equal(g, oc.k_outl):
            bad = np.argwhere(g != oc.k_outl)
            raise AssertionError(f"{what} k_outliers: {len(bad)} mismatches, first at "
                                 f"{bad[0].tolist()}: gpu={g[tuple(bad[0])]:#x} "
                                 f"oracle={oc.k_outl[tuple(bad[0])]:#x}")
    for gname, oname in (("k_res", "k_res"), ("v_res", "v_res")):
        g = getattr(gc, gname)
        if planes is not None:
            g = g[list(planes)]
        g = host(g).view(np.uint16)[:, :, : oc.tr]
        assert np.array_equal(g, getattr(oc, oname)[:, :, : oc.tr]), f"{what} {gname}"


from tests.helpers import row_rel_err  # noqa: E402,F401

ATTN_TOL = 2e-3  # max relative error per output row (fp32 accumulate, fp16 I/O)

"""GPU quantize kernels vs the oracle: codes, scales and zeros bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_bit_kivi_amd import synth
from kv_cache_bit_kivi_amd.cache import KiviCache, make_shape, quantize_k, quantize_v
from tests.gpu_util import announce, assert_cache_equal, dev, host, require_gpu

pytestmark = pytest.mark.gpu


def gpu_quant(fn, x, bits, G, cap, ntok, dst, prev=None):
    B, H, T, D = x.shape
    shape = make_shape(B, H, 1, D, bits, G, max(G, 32), cap)
    if fn is quantize_k:
        codes = torch.zeros((B, H, cap, D * bits // 32), dtype=torch.int32, device="cuda")
        sc = torch.zeros((B, H, cap // G, D), dtype=torch.float32, device="cuda")
    else:
        codes = torch.zeros((B, H, cap // 64, D, 2 * bits), dtype=torch.int32, device="cuda")
        sc = torch.zeros((B, H, cap, D // G), dtype=torch.float32, device="cuda")
    zr = torch.zeros_like(sc)
    fn(shape, dev(x), ntok, dst, codes, sc, zr)
    return host(codes), host(sc), host(zr)


def compare(x, bits, G, cap, ntok, dst, what):
    for gfn, ofn in ((quantize_k, oracle.quantize_k), (quantize_v, oracle.quantize_v)):
        gc, gs, gz = gpu_quant(gfn, x, bits, G, cap, ntok, dst)
        oc, os_, oz = ofn(x, bits, G, cap, ntok, dst)
        name = f"{what} {gfn.__name__}"
        assert np.array_equal(gc, oc), name + " codes"
        assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), name + " scale"
        assert np.array_equal(gz.view(np.uint32), oz.view(np.uint32)), name + " zero"


CASES = [
    # bits, B, H, D, G, T_in, ntok, dst, cap
    (2, 1, 1, 128, 32, 512, 512, 0, 512),
    (4, 1, 1, 128, 32, 512, 512, 0, 512),
    (2, 2, 3, 64, 32, 96, 96, 32, 192),
    (4, 2, 3, 64, 64, 200, 128, 64, 256),
    (2, 3, 2, 32, 32, 64, 32, 96, 128),
    (4, 1, 2, 256, 128, 256, 256, 128, 384),
    (2, 2, 2, 256, 64, 128, 64, 192, 256),
    (2, 1, 4, 128, 128, 384, 384, 0, 384),
    (1, 1, 2, 128, 32, 512, 512, 0, 512),
    (3, 1, 2, 128, 32, 512, 512, 0, 512),
    (1, 2, 3, 64, 32, 96, 96, 32, 192),
    (3, 2, 3, 64, 64, 200, 128, 64, 256),
    (3, 3, 2, 32, 32, 64, 32, 96, 128),
    (1, 1, 2, 256, 128, 256, 256, 128, 384),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b%d_B%dH%dD%dG%d_n%d_o%d" % (
    c[0], c[1], c[2], c[3], c[4], c[6], c[7]))
def test_quantize_random_shapes(case):
    require_gpu()
    bits, B, H, D, G, T, ntok, dst, cap = case
    announce(f"quantize {case}")
    x = synth.random_fp16(hash(case) % 10000, (B, H, T, D), scale=2.0)
    x[..., 1] *= np.float16(10)
    compare(x, bits, G, cap, ntok, dst, str(case))


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("lo,hi", [(-65504.0, 65504.0), (-1.0, 1.0), (0.0, 2.0 ** -14),
                                   (-3.0, -2.0 ** -20), (1000.0, 1024.0)])
def test_exhaustive_fp16_values(bits, lo, hi):
    """Every finite fp16 value in [lo, hi] goes through both quantizers in
    groups whose minimum is lo and maximum is hi."""
    require_gpu()
    announce(f"exhaustive fp16 bits={bits} [{lo}, {hi}]")
    allv = np.arange(65536, dtype=np.uint16).view(np.float16)
    f = allv.astype(np.float32)
    sel = np.isfinite(f) & (f >= np.float32(lo)) & (f <= np.float32(hi))
    vals = allv[sel]
    G, D = 32, 128
    per = G - 2
    ngroups = (len(vals) + per - 1) // per
    pad = np.full(ngroups * per, np.float16(lo), np.float16)
    pad[: len(vals)] = vals
    groups = np.empty((ngroups, G), np.float16)
    groups[:, 0] = np.float16(lo)
    groups[:, 1] = np.float16(hi)
    groups[:, 2:] = pad.reshape(ngroups, per)
    # keys: groups run down a channel (G tokens); values: along a token's channels
    nk = (ngroups + D - 1) // D
    gk = np.full((nk * D, G), np.float16(lo), np.float16)
    gk[:ngroups] = groups
    k = gk.reshape(nk, D, G).transpose(0, 2, 1).reshape(1, 1, nk * G, D)
    T = nk * G
    cap = (T + 63) // 64 * 64
    for gfn, ofn in ((quantize_k, oracle.quantize_k),):
        gc, gs, gz = gpu_quant(gfn, k, bits, G, cap, T, 0)
        oc, os_, oz = ofn(k, bits, G, cap, T, 0)
        assert np.array_equal(gc, oc) and np.array_equal(gs.view(np.uint32), os_.view(np.uint32))
        assert np.array_equal(gz.view(np.uint32), oz.view(np.uint32))
    nv = (ngroups + 3) // 4                 # 4 groups per 128-channel token
    nv = (nv + 31) // 32 * 32
    gv = np.full((nv * 4, G), np.float16(lo), np.float16)
    gv[:ngroups] = groups
    v = gv.reshape(1, 1, nv, D)
    capv = (nv + 63) // 64 * 64
    gc, gs, gz = gpu_quant(quantize_v, v, bits, G, capv, nv, 0)
    oc, os_, oz = oracle.quantize_v(v, bits, G, capv, nv, 0)
    assert np.array_equal(gc, oc) and np.array_equal(gs.view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(gz.view(np.uint32), oz.view(np.uint32))


def test_signed_zero_and_constant_groups():
    """+0/-0 ties (the first extremum in index order is kept), constant
    groups and groups spanning a single ulp."""
    require_gpu()
    announce("signed zeros / constant groups")
    G, D, T = 32, 64, 128
    x = np.zeros((1, 2, T, D), np.float16)
    x[0, 0, 0::2, :] = np.float16(-0.0)        # alternate -0 / +0
    x[0, 1, :, :] = np.float16(0.0)
    x[0, 1, 5, :] = np.float16(-0.0)
    x[0, 1, 32:64, :] = np.float16(3.0)         # constant group
    x[0, 1, 64:96, 3] = np.float16(1.0)
    x[0, 1, 70, 3] = np.nextafter(np.float16(1.0), np.float16(2.0))
    x[0, 0, :, 1::2] = np.float16(-0.0)
    for bits in (1, 2, 3, 4):
        compare(x, bits, G, T, T, 0, "zeros")


@pytest.mark.parametrize("name,batches", [
    ("single_head_512", None),
    ("llama2_7b_b8_ctx4096", [0, 5]),
    ("mistral_7b_b32_ctx8192", [3, 31]),
    ("stream_b64_4bit", [0, 63]),
])
def test_prefill_workloads(name, batches):
    """Full-size prefill of each workload on the GPU; the oracle checks the
    listed batch entries (every head, every token) bit-exactly."""
    require_gpu()
    w = synth.WORKLOADS[name]
    announce(f"prefill {name}")
    k, v = synth.kv(w)
    gc = KiviCache(w.batch, w.kv_heads, w.gqa, w.head_dim, w.bits, w.group, w.residual,
                   w.capacity())
    gc.prefill(dev(k), dev(v), w.tq)
    sel = list(range(w.batch)) if batches is None else batches
    oc = oracle.OracleCache(len(sel), w.kv_heads, w.gqa, w.head_dim, w.bits, w.group,
                            w.residual, w.capacity())
    oc.prefill(k[sel], v[sel], w.tq)
    assert_cache_equal(gc, oc, planes=sel, what=name)

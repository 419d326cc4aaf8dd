"""1- and 3-bit codes beyond the codec and attention tests: the fused step
equals the separate calls bit for bit and meets the oracle, ragged and paged
caches equal their references, and the batch-8 Llama-2-7B-shaped layer at
full size (prefill bit-exact against the oracle, every decode row within the
bar).  Comparisons of two calls bit for bit use deterministic caches."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_bit_kivi_amd import synth
from kv_cache_bit_kivi_amd.cache import KiviCache, PagedKiviCache, RaggedKiviCache
from tests.gpu_util import (ATTN_TOL, announce, assert_cache_equal, dev, host, require_gpu,
                            row_rel_err)

pytestmark = pytest.mark.gpu

SCALE = 0.0883883461356163


@pytest.mark.parametrize("bits", [1, 3])
@pytest.mark.parametrize("r,D,S", [(1, 128, 0), (4, 128, 3), (2, 64, 0)])
def test_fused_stream(bits, r, D, S):
    require_gpu()
    announce(f"fused stream bits={bits} r={r} D={D} S={S}")
    B, H, G, R = 2, 2, 32, 32
    tq0, tr0, steps = 128, 29, R + 6
    T = tq0 + tr0 + steps
    k = synth.random_fp16(800 + bits + r, (B, H, T, D), scale=2.0)
    k[..., 3] *= np.float16(10)
    v = synth.random_fp16(810 + bits + r, (B, H, T, D))
    qs = synth.random_fp16(820 + bits + r, (steps, B, H * r, D))
    cap = (T + R + 63) // 64 * 64
    sep = KiviCache(B, H, r, D, bits, G, R, cap, deterministic=True)
    fus = KiviCache(B, H, r, D, bits, G, R, cap, deterministic=True)
    oc = oracle.OracleCache(B, H, r, D, bits, G, R, cap)
    kd, vd = dev(k[:, :, : tq0 + tr0]), dev(v[:, :, : tq0 + tr0])
    sep.prefill(kd, vd, tq0)
    fus.prefill(kd, vd, tq0)
    oc.prefill(k[:, :, : tq0 + tr0], v[:, :, : tq0 + tr0], tq0)
    for i in range(steps):
        t = tq0 + tr0 + i
        kn, vn = np.ascontiguousarray(k[:, :, t]), np.ascontiguousarray(v[:, :, t])
        q = dev(qs[i])
        sep.append(dev(kn), dev(vn))
        o_sep = host(sep.decode(q, SCALE, num_splits=S))
        o_fus = host(fus.append_decode(dev(kn), dev(vn), q, SCALE, num_splits=S))
        assert np.array_equal(o_fus.view(np.uint16), o_sep.view(np.uint16)), f"step {i}"
        oc.append(kn, vn)
        if i in (0, 3, R + 5):
            assert_cache_equal(fus, oc, what=f"step {i}")
        err = row_rel_err(o_fus.astype(np.float64), oc.decode(np.ascontiguousarray(qs[i]), SCALE))
        assert err <= ATTN_TOL, (i, err)
    assert oc.flushes == 2


@pytest.mark.parametrize("bits", [1, 3])
def test_ragged_and_paged(bits):
    """Ragged caches meet per-sequence oracle replays; a paged cache with a
    shuffled table gives the ragged cache's outputs bit for bit."""
    require_gpu()
    announce(f"ragged + paged bits={bits}")
    B, H, r, D, G, R, P = 3, 2, 2, 128, 32, 32, 64
    ctx = [70, 400, 33]
    tq = [c - ((c - 1) % R + 1) for c in ctx]
    steps = R + 2
    cap = 640
    T = max(ctx) + steps
    k = synth.random_fp16(900 + bits, (B, H, T, D), scale=2.0)
    v = synth.random_fp16(910 + bits, (B, H, T, D))
    qs = synth.random_fp16(920 + bits, (steps + 1, B, H * r, D))
    rc = RaggedKiviCache(B, H, r, D, bits, G, R, cap, deterministic=True)
    table = np.random.default_rng(bits).permutation(B * (cap // P)).astype(np.int32)
    pc = PagedKiviCache(B, H, r, D, bits, G, R, cap, P, table=table.reshape(B, cap // P),
                        deterministic=True)
    kd, vd = dev(k), dev(v)
    rc.prefill(kd, vd, ctx, tq)
    pc.prefill(kd, vd, ctx, tq)
    ocs = []
    for b in range(B):
        oc = oracle.OracleCache(1, H, r, D, bits, G, R, cap)
        oc.prefill(k[b:b + 1, :, : ctx[b]], v[b:b + 1, :, : ctx[b]], tq[b])
        ocs.append(oc)
    for i in range(steps):
        kn = np.stack([k[b, :, ctx[b] + i] for b in range(B)])
        vn = np.stack([v[b, :, ctx[b] + i] for b in range(B)])
        q = dev(qs[i])
        a = host(rc.append_decode(dev(kn), dev(vn), q, SCALE))
        p = host(pc.append_decode(dev(kn), dev(vn), q, SCALE))
        assert np.array_equal(a.view(np.uint16), p.view(np.uint16)), f"step {i}"
        for b, oc in enumerate(ocs):
            oc.append(np.ascontiguousarray(kn[b:b + 1]), np.ascontiguousarray(vn[b:b + 1]))
            ref = oc.decode(np.ascontiguousarray(qs[i][b:b + 1]), SCALE)
            assert row_rel_err(a[b:b + 1].astype(np.float64), ref) <= ATTN_TOL, (i, b)
    for name in ("k_codes", "k_scale", "v_codes", "v_zero"):
        g = pc.gather(name)
        rr = host(getattr(rc, name))
        assert np.array_equal(g.view(np.uint32), rr.view(np.uint32)), name


@pytest.mark.parametrize("bits", [1, 3])
def test_workload_full_size(bits):
    """The batch-8 Llama-2-7B-shaped layer at 1 and 3 bits: prefill bit-exact
    on two batch entries, decode of every row within the bar."""
    require_gpu()
    w = synth.WORKLOADS["llama2_7b_b8_ctx4096"].with_(bits=bits)
    announce(f"workload llama2_7b_b8_ctx4096 bits={bits}")
    k, v = synth.kv(w)
    q = synth.query(w)
    gc = KiviCache(w.batch, w.kv_heads, w.gqa, w.head_dim, w.bits, w.group, w.residual,
                   w.capacity())
    gc.prefill(dev(k), dev(v), w.tq)
    out = host(gc.decode(dev(q), w.softmax_scale)).astype(np.float64)
    sel = [0, 5]
    oc = oracle.OracleCache(len(sel), w.kv_heads, w.gqa, w.head_dim, w.bits, w.group, w.residual,
                            w.capacity())
    oc.prefill(k[sel], v[sel], w.tq)
    assert_cache_equal(gc, oc, planes=sel, what="prefill")
    full = oracle.OracleCache(w.batch, w.kv_heads, w.gqa, w.head_dim, w.bits, w.group,
                              w.residual, w.capacity())
    full.prefill(k, v, w.tq)
    err = row_rel_err(out, full.decode(q, w.softmax_scale))
    assert err <= ATTN_TOL, err
    torch.cuda.synchronize()

"""Pre-RoPE keys on the GPU against the oracle.

Page: "KVQuant: Towards 10 Million Context Length LLM Inference with KV Cache
Quantization" (codewithpapers.app, abstract): keys are quantized before the
rotary positional embedding.  The cache stores pre-RoPE keys; decode rotates
each key at its token index (rotate-half pairs, frequency theta^(-2i/D)).
Bar: the quantized store bit-exact (it does not depend on the embedding);
attention within the row bar on the matrix-core kernel's pre-RoPE variant
(lane-per-token key scores) and on the generic kernel, over split counts,
positions up to 64K, ragged and paged stores, the fused step and the
full-size Llama-2-7B-shaped layer.  Comparisons of two calls bit for bit use
deterministic caches."""
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


def keys(seed, shape):
    k = synth.random_fp16(seed, shape, scale=2.0)
    k[..., 5] *= np.float16(10)
    k[..., shape[-1] // 2 + 6] *= np.float16(8)     # a large channel in the second half
    return k


def build(B, H, r, D, bits, G, R, tq, tr, theta, mh, seed, n_out=0, deterministic=False):
    L = tq + tr
    cap = max(64, (tq + 2 * R + 63) // 64 * 64)
    cap = (cap + G - 1) // G * G
    k = keys(seed, (B, H, L, D))
    v = synth.random_fp16(seed + 1, (B, H, L, D))
    q = synth.random_fp16(seed + 2, (B, H * r, D))
    gc = KiviCache(B, H, r, D, bits, G, R, cap, meta_half=mh, outliers=n_out, rope_theta=theta,
                   deterministic=deterministic)
    gc.prefill(dev(k), dev(v), tq)
    oc = oracle.OracleCache(B, H, r, D, bits, G, R, cap, meta_half=mh, n_out=n_out,
                            rope_theta=theta)
    oc.prefill(k, v, tq)
    return gc, oc, k, v, q


SHAPES = [
    # B, H, r, D, bits, G, R, tq, tr, theta, meta_half, n_out
    (2, 2, 1, 128, 2, 32, 128, 992, 128, 10000.0, False, 0),     # matrix-core, half tile
    (2, 2, 1, 128, 1, 32, 128, 1024, 77, 10000.0, True, 0),
    (1, 3, 2, 128, 3, 32, 64, 1472, 9, 500000.0, False, 0),
    (1, 3, 4, 128, 4, 32, 128, 2016, 100, 10000.0, False, 0),    # (the 4-wave variant)
    (1, 2, 4, 128, 2, 32, 128, 1536, 60, 10000.0, True, 0),
    (1, 2, 8, 128, 2, 32, 128, 512, 40, 10000.0, False, 0),
    (2, 1, 2, 128, 4, 32, 32, 640, 32, 1000000.0, True, 0),
    (1, 2, 1, 128, 2, 32, 128, 0, 97, 10000.0, False, 0),        # residual only
    (2, 2, 2, 64, 4, 64, 128, 448, 1, 10000.0, False, 0),        # generic kernel
    (3, 1, 1, 32, 2, 32, 32, 96, 31, 10000.0, True, 0),          # generic kernel
    (1, 2, 1, 128, 2, 32, 128, 1024, 50, 10000.0, False, 1),     # generic (rope + outliers)
]


@pytest.mark.parametrize("shp", SHAPES, ids=lambda s: "B%dH%dr%dD%db%dG%dR%d_tq%d_tr%d_th%g" % s[:10]
                         + ("_m16" if s[10] else "") + (f"_k{s[11]}" if s[11] else ""))
@pytest.mark.parametrize("splits", [0, 1, 5])
def test_decode_rope(shp, splits):
    require_gpu()
    B, H, r, D, bits, G, R, tq, tr, theta, mh, n_out = shp
    announce(f"decode rope {shp} splits={splits}")
    gc, oc, k, v, q = build(B, H, r, D, bits, G, R, tq, tr, theta, mh, seed=sum(shp[:9]),
                            n_out=n_out)
    assert_cache_equal(gc, oc, what="prefill")
    ref = oc.decode(q, SCALE)
    out = host(gc.decode(dev(q), SCALE, num_splits=splits)).astype(np.float64)
    err = row_rel_err(out, ref)
    assert err <= ATTN_TOL, err


@pytest.mark.parametrize("splits", [1, 7])
def test_decode_rope_long_positions(splits):
    """Positions up to 65,536: the per-wave angle recurrence and the split
    starts at large positions keep the rotation exact enough."""
    require_gpu()
    announce(f"decode rope long positions splits={splits}")
    gc, oc, k, v, q = build(1, 2, 1, 128, 2, 32, 128, 65408, 128, 10000.0, False, seed=71)
    ref = oc.decode(q, SCALE)
    out = host(gc.decode(dev(q), SCALE, num_splits=splits)).astype(np.float64)
    assert row_rel_err(out, ref) <= ATTN_TOL


@pytest.mark.parametrize("r", [1, 2])
def test_decode_rope_deterministic(r):
    """A deterministic cache repeats its bits; the default (shared tiles)
    stays within the bar on every call."""
    require_gpu()
    announce(f"decode rope deterministic r={r}")
    gc, oc, k, v, q = build(2, 4, r, 128, 2, 32, 128, 2048, 60, 10000.0, False, seed=5,
                            deterministic=True)
    qd = dev(q)
    a = host(gc.decode(qd, SCALE))
    for _ in range(3):
        assert np.array_equal(a.view(np.uint16), host(gc.decode(qd, SCALE)).view(np.uint16))
    gs, _, _, _, _ = build(2, 4, r, 128, 2, 32, 128, 2048, 60, 10000.0, False, seed=5)
    ref = oc.decode(q, SCALE)
    for _ in range(3):
        assert row_rel_err(host(gs.decode(qd, SCALE)).astype(np.float64), ref) <= ATTN_TOL


@pytest.mark.parametrize("bits,r", [(2, 1), (4, 4), (1, 2), (3, 8)])
def test_stream_rope_fused(bits, r):
    """Appends through flushes: the fused step equals append + decode bit for
    bit, the store equals the oracle's, attention within the bar (positions
    keep counting across flushes)."""
    require_gpu()
    announce(f"stream rope bits={bits} r={r}")
    B, H, D, G, R = 2, 2, 128, 32, 32
    tq0, tr0, n = 128, 30, 2 * R + 5
    T = tq0 + tr0 + n
    seed = 500 + 10 * bits + r
    k = keys(seed, (B, H, T, D))
    v = synth.random_fp16(seed + 1, (B, H, T, D))
    qs = synth.random_fp16(seed + 2, (n, B, H * r, D))
    cap = (T + R + 63) // 64 * 64
    sep = KiviCache(B, H, r, D, bits, G, R, cap, rope_theta=10000.0, deterministic=True)
    fus = KiviCache(B, H, r, D, bits, G, R, cap, rope_theta=10000.0, deterministic=True)
    oc = oracle.OracleCache(B, H, r, D, bits, G, R, cap, rope_theta=10000.0)
    kd, vd = dev(k[:, :, : tq0 + tr0]), dev(v[:, :, : tq0 + tr0])
    sep.prefill(kd, vd, tq0)
    fus.prefill(kd, vd, tq0)
    oc.prefill(k[:, :, : tq0 + tr0], v[:, :, : tq0 + tr0], tq0)
    for i in range(n):
        t = tq0 + tr0 + i
        kn, vn = np.ascontiguousarray(k[:, :, t]), np.ascontiguousarray(v[:, :, t])
        q = dev(qs[i])
        sep.append(dev(kn), dev(vn))
        o_sep = host(sep.decode(q, SCALE))
        o_fus = host(fus.append_decode(dev(kn), dev(vn), q, SCALE))
        assert np.array_equal(o_fus.view(np.uint16), o_sep.view(np.uint16)), f"step {i}"
        oc.append(kn, vn)
        if i in (0, R + 2, n - 1):
            assert_cache_equal(fus, oc, what=f"fused step {i}")
        ref = oc.decode(np.ascontiguousarray(qs[i]), SCALE)
        err = row_rel_err(o_fus.astype(np.float64), ref)
        assert err <= ATTN_TOL, (i, err)
    assert oc.flushes == 3


@pytest.mark.parametrize("case", [
    # B, H, r, D, bits, G, R, ntok, tq
    (4, 2, 1, 128, 2, 32, 128, [69, 1152, 320, 2125], [64, 1024, 320, 2048]),
    (3, 2, 4, 128, 4, 32, 64, [100, 700, 1500], [64, 640, 1472]),
    (3, 2, 2, 64, 2, 32, 32, [60, 300, 2], [32, 288, 0]),        # generic kernel
], ids=lambda c: "B%dH%dr%dD%db%dG%dR%d" % c[:7])
def test_ragged_rope(case):
    """Each sequence of a ragged cache counts positions from its own start."""
    require_gpu()
    B, H, r, D, bits, G, R, ntok, tq = case
    announce(f"ragged rope {case}")
    cap = max(64, (max(tq) + 2 * R + 63) // 64 * 64)
    T = max(ntok)
    k = keys(sum(ntok), (B, H, T, D))
    v = synth.random_fp16(sum(ntok) + 1, (B, H, T, D))
    q = synth.random_fp16(sum(ntok) + 2, (B, H * r, D))
    gc = RaggedKiviCache(B, H, r, D, bits, G, R, cap, rope_theta=10000.0)
    gc.prefill(dev(k), dev(v), ntok, tq)
    for splits in (0, 3):
        out = host(gc.decode(dev(q), SCALE, num_splits=splits))
        for b in range(B):
            oc = oracle.OracleCache(1, H, r, D, bits, G, R, cap, rope_theta=10000.0)
            oc.prefill(k[b:b + 1, :, : ntok[b]], v[b:b + 1, :, : ntok[b]], tq[b])
            ref = oc.decode(np.ascontiguousarray(q[b:b + 1]), SCALE)
            err = row_rel_err(out[b:b + 1].astype(np.float64), ref)
            assert err <= ATTN_TOL, (splits, b, err)


def test_paged_rope():
    """A paged store with pre-RoPE keys (shuffled table) gives the ragged
    store's outputs bit for bit through appends and flushes."""
    require_gpu()
    announce("paged rope")
    B, H, r, D, bits, G, R, P = 3, 2, 2, 128, 2, 32, 32, 64
    ctx = [200, 40, 129]
    tq = [c - ((c - 1) % R + 1) for c in ctx]
    steps = R + 3
    cap = ((max(tq) + (steps // R + 2) * R + P - 1) // P) * P
    mp = cap // P
    table = np.random.default_rng(4).permutation(B * mp + 3)[: B * mp].astype(np.int32)
    T = max(ctx) + steps
    k = keys(61, (B, H, T, D))
    v = synth.random_fp16(62, (B, H, T, D))
    rc = RaggedKiviCache(B, H, r, D, bits, G, R, cap, rope_theta=10000.0, deterministic=True)
    pc = PagedKiviCache(B, H, r, D, bits, G, R, cap, P, num_pages=B * mp + 3,
                        table=table.reshape(B, mp), rope_theta=10000.0, deterministic=True)
    rc.prefill(dev(k), dev(v), ctx, tq)
    pc.prefill(dev(k), dev(v), ctx, tq)
    for i in range(steps):
        kn = dev(np.stack([k[b, :, ctx[b] + i] for b in range(B)]))
        vn = dev(np.stack([v[b, :, ctx[b] + i] for b in range(B)]))
        q = dev(synth.random_fp16(70 + i, (B, H * r, D)))
        a = host(rc.append_decode(kn, vn, q, SCALE))
        b_ = host(pc.append_decode(kn, vn, q, SCALE))
        assert np.array_equal(a.view(np.uint16), b_.view(np.uint16)), i


def test_decode_rope_workload():
    """The batch-8 Llama-2-7B-shaped layer (32 heads, head_dim 128, 3968
    quantized + 128 residual tokens, 2-bit, G = 32) with pre-RoPE keys
    (theta 10000): every decode row within the bar."""
    require_gpu()
    w = synth.WORKLOADS["llama2_7b_b8_ctx4096"]
    announce("decode rope llama2_7b_b8_ctx4096")
    k, v = synth.kv(w)
    q = synth.query(w)
    gc = KiviCache(w.batch, w.kv_heads, w.gqa, w.head_dim, w.bits, w.group, w.residual,
                   w.capacity(), rope_theta=10000.0)
    gc.prefill(dev(k), dev(v), w.tq)
    out = host(gc.decode(dev(q), w.softmax_scale)).astype(np.float64)
    oc = oracle.OracleCache(w.batch, w.kv_heads, w.gqa, w.head_dim, w.bits, w.group,
                            w.residual, w.capacity(), rope_theta=10000.0)
    oc.prefill(k, v, w.tq)
    ref = oc.decode(q, w.softmax_scale)
    err = row_rel_err(out, ref)
    assert err <= ATTN_TOL, err
    torch.cuda.synchronize()

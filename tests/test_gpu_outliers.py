"""Key outlier isolation (dense-and-sparse keys) on the GPU against the
oracle.

Page: "KVQuant: Towards 10 Million Context Length LLM Inference with KV Cache
Quantization" (codewithpapers.app, abstract): outliers are isolated per
vector.  Bar: codes, scales, zeros and the sparse outlier words bit-exact
(quantize, prefill, flushes; contiguous, ragged and paged stores); attention
within the row bar on the matrix-core kernel (1 or 2 outliers per group) and
the generic kernel (any count); the fused step equal to the separate calls;
repeated decodes bit-identical; the full-size Llama-2-7B-shaped layer."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_bit_kivi_amd import synth
from kv_cache_bit_kivi_amd.cache import (KiviCache, PagedKiviCache, RaggedKiviCache, make_shape,
                                         quantize_k)
from tests.gpu_util import (ATTN_TOL, announce, assert_cache_equal, dev, host, require_gpu,
                            row_rel_err)

pytestmark = pytest.mark.gpu

SCALE = 0.0883883461356163


def gpu_quant_k(x, bits, G, cap, ntok, dst, n_out, mh):
    B, H, T, D = x.shape
    shape = make_shape(B, H, 1, D, bits, G, max(G, 32), cap, meta_half=mh, outliers=n_out)
    mdt = torch.float16 if mh else torch.float32
    codes = torch.zeros((B, H, cap, D * bits // 32), dtype=torch.int32, device="cuda")
    sc = torch.zeros((B, H, cap // G, D), dtype=mdt, device="cuda")
    zr = torch.zeros_like(sc)
    outl = torch.zeros((B, H, cap // G, n_out, D), dtype=torch.int32, device="cuda")
    quantize_k(shape, dev(x), ntok, dst, codes, sc, zr, outl)
    return host(codes), host(sc), host(zr), host(outl)


def compare_k(x, bits, G, cap, ntok, dst, n_out, mh, what):
    gc, gs, gz, go = gpu_quant_k(x, bits, G, cap, ntok, dst, n_out, mh)
    oc, os_, oz, oo = oracle.quantize_k(x, bits, G, cap, ntok, dst, meta_half=mh, n_out=n_out)
    bits_t = np.uint16 if mh else np.uint32
    for name, g, o in (("outliers", go, oo), ("codes", gc, oc),
                       ("scale", gs.view(bits_t), os_.view(bits_t)),
                       ("zero", gz.view(bits_t), oz.view(bits_t))):
        if not np.array_equal(g, o):
            bad = np.argwhere(g != o)
            raise AssertionError(f"{what} {name}: {len(bad)} mismatches, first at "
                                 f"{bad[0].tolist()}: gpu={g[tuple(bad[0])]} "
                                 f"oracle={o[tuple(bad[0])]}")


CODEC_CASES = [
    # bits, B, H, D, G, T_in, ntok, dst, cap, n_out, meta_half
    (2, 1, 2, 128, 32, 512, 512, 0, 512, 1, False),
    (4, 1, 2, 128, 32, 256, 256, 0, 256, 2, True),
    (1, 2, 3, 64, 32, 96, 96, 32, 192, 3, False),
    (3, 2, 3, 64, 64, 200, 128, 64, 256, 8, True),
    (4, 1, 2, 256, 128, 256, 256, 128, 384, 5, False),
    (3, 1, 2, 128, 32, 64, 64, 0, 64, 8, False),
]


@pytest.mark.parametrize("case", CODEC_CASES, ids=lambda c: "b%d_B%dH%dD%dG%d_n%d_o%d_k%d%s" % (
    c[0], c[1], c[2], c[3], c[4], c[6], c[7], c[9], "_m16" if c[10] else ""))
def test_quantize_outliers(case):
    require_gpu()
    bits, B, H, D, G, T, ntok, dst, cap, n_out, mh = case
    announce(f"quantize outliers {case}")
    x = synth.spiky_fp16(sum(case[:10]), (B, H, T, D), rate=0.03, scale=2.0)
    compare_k(x, bits, G, cap, ntok, dst, n_out, mh, str(case))


@pytest.mark.parametrize("n_out", [1, 2, 7])
def test_quantize_outliers_ties(n_out):
    """Magnitude ties everywhere (small integers of both signs, all-zero and
    signed-zero columns, constant columns): the lower token wins each tie."""
    require_gpu()
    announce(f"quantize outliers ties n_out={n_out}")
    rng = np.random.default_rng(40 + n_out)
    G, D, T = 32, 128, 128
    x = rng.integers(-4, 5, (2, 2, T, D)).astype(np.float16)
    x[0, 0, :, 3] = 0
    x[0, 1, :, 4] = np.float16(-0.0)
    x[1, 0, :, 5] = 7
    x[1, 1, ::2, 6] = -3
    x[1, 1, 1::2, 6] = 3
    for bits in (1, 2, 3, 4):
        compare_k(x, bits, G, T, T, 0, n_out, False, f"ties bits={bits}")


def build(B, H, r, D, bits, G, R, tq, tr, n_out, mh, seed, cls=KiviCache, deterministic=False):
    L = tq + tr
    cap = max(64, (tq + 2 * R + 63) // 64 * 64)
    cap = (cap + G - 1) // G * G
    k = synth.spiky_fp16(seed, (B, H, L, D), rate=0.02, scale=2.0)
    v = synth.random_fp16(seed + 1, (B, H, L, D))
    q = synth.random_fp16(seed + 2, (B, H * r, D))
    gc = KiviCache(B, H, r, D, bits, G, R, cap, meta_half=mh, outliers=n_out,
                   deterministic=deterministic)
    gc.prefill(dev(k), dev(v), tq)
    oc = oracle.OracleCache(B, H, r, D, bits, G, R, cap, meta_half=mh, n_out=n_out)
    oc.prefill(k, v, tq)
    return gc, oc, k, v, q


SHAPES = [
    # B, H, r, D, bits, G, R, tq, tr, n_out, meta_half
    (2, 2, 1, 128, 2, 32, 128, 992, 128, 1, False),     # matrix-core kernel, half tile
    (2, 2, 1, 128, 2, 32, 128, 1024, 77, 2, True),
    (1, 3, 4, 128, 4, 32, 128, 2016, 100, 1, False),
    (1, 2, 8, 128, 2, 32, 128, 512, 40, 2, False),
    (2, 1, 2, 128, 1, 32, 32, 640, 32, 1, True),
    (1, 2, 1, 128, 3, 32, 64, 1472, 9, 2, False),
    (2, 2, 2, 64, 4, 64, 128, 448, 1, 3, False),        # generic kernel
    (1, 2, 1, 128, 2, 32, 128, 1024, 50, 4, True),      # generic kernel (4 outliers)
    (3, 1, 1, 32, 2, 32, 32, 96, 31, 8, False),         # generic kernel
]


@pytest.mark.parametrize("shp", SHAPES, ids=lambda s: "B%dH%dr%dD%db%dG%dR%d_tq%d_tr%d_k%d" % s[:10]
                         + ("_m16" if s[10] else ""))
@pytest.mark.parametrize("splits", [0, 1, 5])
def test_decode_outliers(shp, splits):
    require_gpu()
    B, H, r, D, bits, G, R, tq, tr, n_out, mh = shp
    announce(f"decode outliers {shp} splits={splits}")
    gc, oc, k, v, q = build(B, H, r, D, bits, G, R, tq, tr, n_out, mh, seed=sum(shp[:10]))
    assert_cache_equal(gc, oc, what="prefill")
    ref = oc.decode(q, SCALE)
    out = host(gc.decode(dev(q), SCALE, num_splits=splits)).astype(np.float64)
    err = row_rel_err(out, ref)
    assert err <= ATTN_TOL, err


@pytest.mark.parametrize("n_out,r", [(1, 8), (2, 1), (2, 4)])
def test_decode_outliers_deterministic(n_out, r):
    """Two identical calls with outlier corrections give identical bits."""
    require_gpu()
    announce(f"decode outliers deterministic n_out={n_out} r={r}")
    gc, oc, k, v, q = build(2, 4, r, 128, 2, 32, 128, 2048, 60, n_out, False, seed=5 + r,
                            deterministic=True)
    qd = dev(q)
    a = host(gc.decode(qd, SCALE))
    for _ in range(3):
        b = host(gc.decode(qd, SCALE))
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("n_out,r", [(1, 1), (2, 4), (3, 2)])
def test_stream_outliers_fused(bits, n_out, r):
    """Appends through flushes: the fused step equals append + decode bit for
    bit, every cache buffer (outlier words included) equals the oracle's."""
    require_gpu()
    announce(f"stream outliers bits={bits} n_out={n_out} r={r}")
    B, H, D, G, R = 2, 2, 128, 32, 32
    tq0, tr0, n = 128, 30, 2 * R + 5
    T = tq0 + tr0 + n
    seed = 300 + 10 * bits + n_out + r
    k = synth.spiky_fp16(seed, (B, H, T, D), rate=0.03, scale=1.5)
    v = synth.random_fp16(seed + 1, (B, H, T, D))
    qs = synth.random_fp16(seed + 2, (n, B, H * r, D))
    cap = (T + R + 63) // 64 * 64
    sep = KiviCache(B, H, r, D, bits, G, R, cap, outliers=n_out, deterministic=True)
    fus = KiviCache(B, H, r, D, bits, G, R, cap, outliers=n_out, deterministic=True)
    oc = oracle.OracleCache(B, H, r, D, bits, G, R, cap, n_out=n_out)
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
        if i in (0, 2, R + 2, n - 1):
            assert_cache_equal(fus, oc, what=f"fused step {i}")
            assert_cache_equal(sep, oc, what=f"separate step {i}")
        ref = oc.decode(np.ascontiguousarray(qs[i]), SCALE)
        err = row_rel_err(o_fus.astype(np.float64), ref)
        assert err <= ATTN_TOL, (i, err)
    assert oc.flushes == 3


def _seq_oracles(k, v, ntok, tq, H, r, D, bits, G, R, cap, n_out, mh):
    ocs = []
    for b in range(len(ntok)):
        oc = oracle.OracleCache(1, H, r, D, bits, G, R, cap, meta_half=mh, n_out=n_out)
        oc.prefill(k[b:b + 1, :, : ntok[b]], v[b:b + 1, :, : ntok[b]], tq[b])
        ocs.append(oc)
    return ocs


@pytest.mark.parametrize("case", [
    # B, H, r, D, bits, G, R, ntok, tq, n_out, meta_half
    (4, 2, 1, 128, 2, 32, 128, [69, 1152, 320, 2125], [64, 1024, 320, 2048], 1, False),
    (3, 2, 4, 128, 4, 32, 64, [100, 700, 1500], [64, 640, 1472], 2, True),
    (3, 2, 2, 64, 2, 32, 32, [60, 300, 2], [32, 288, 0], 2, False),      # generic kernel
], ids=lambda c: "B%dH%dr%dD%db%dG%dR%d_k%d" % (c[:7] + (c[9],)))
def test_ragged_outliers(case):
    """Each sequence of a ragged cache with outliers equals a one-sequence
    oracle cache (bit-exact store, attention within the bar), through a
    staggered flush."""
    require_gpu()
    B, H, r, D, bits, G, R, ntok, tq, n_out, mh = case
    announce(f"ragged outliers {case}")
    cap = max(64, (max(tq) + 2 * R + 63) // 64 * 64)
    T = max(ntok) + R + 2
    k = synth.spiky_fp16(sum(ntok), (B, H, T, D), rate=0.02, scale=2.0)
    v = synth.random_fp16(sum(ntok) + 1, (B, H, T, D))
    gc = RaggedKiviCache(B, H, r, D, bits, G, R, cap, meta_half=mh, outliers=n_out)
    gc.prefill(dev(k), dev(v), ntok, tq)
    ocs = _seq_oracles(k, v, ntok, tq, H, r, D, bits, G, R, cap, n_out, mh)
    steps = R + 2
    for i in range(steps + 1):
        q = synth.random_fp16(900 + i, (B, H * r, D))
        if i == 0:
            out = host(gc.decode(dev(q), SCALE))
        else:
            kn = np.stack([k[b, :, ntok[b] + i - 1] for b in range(B)])
            vn = np.stack([v[b, :, ntok[b] + i - 1] for b in range(B)])
            out = host(gc.append_decode(dev(kn), dev(vn), dev(q), SCALE))
            for b, oc in enumerate(ocs):
                oc.append(np.ascontiguousarray(kn[b:b + 1]), np.ascontiguousarray(vn[b:b + 1]))
        if i in (0, steps):
            for b, oc in enumerate(ocs):
                assert (int(gc.tq[b]), int(gc.tr[b])) == (oc.tq, oc.tr)
                g = host(gc.k_outliers[b:b + 1])
                assert np.array_equal(g[:, :, : oc.tq // G], oc.k_outl[:, :, : oc.tq // G]), b
                gcodes = host(gc.k_codes[b:b + 1])[:, :, : oc.tq]
                assert np.array_equal(gcodes, oc.k_codes[:, :, : oc.tq]), b
        for b, oc in enumerate(ocs):
            ref = oc.decode(np.ascontiguousarray(q[b:b + 1]), SCALE)
            err = row_rel_err(out[b:b + 1].astype(np.float64), ref)
            assert err <= ATTN_TOL, (i, b, err)


def test_paged_outliers():
    """A paged store with outliers (permuted table) equals the ragged store:
    gathered outlier words and codes bit-exact, outputs bit-identical."""
    require_gpu()
    announce("paged outliers")
    B, H, r, D, bits, G, R, P, n_out = 3, 2, 2, 128, 2, 32, 32, 64, 2
    ctx = [200, 40, 129]
    tq = [c - ((c - 1) % R + 1) for c in ctx]
    steps = R + 3
    cap = ((max(tq) + (steps // R + 2) * R + P - 1) // P) * P
    mp = cap // P
    rng = np.random.default_rng(3)
    table = rng.permutation(B * mp + 4)[: B * mp].astype(np.int32).reshape(B, mp)
    T = max(ctx) + steps
    k = synth.spiky_fp16(31, (B, H, T, D), rate=0.03, scale=2.0)
    v = synth.random_fp16(32, (B, H, T, D))
    rc = RaggedKiviCache(B, H, r, D, bits, G, R, cap, outliers=n_out, deterministic=True)
    pc = PagedKiviCache(B, H, r, D, bits, G, R, cap, P, num_pages=B * mp + 4, table=table,
                        outliers=n_out, deterministic=True)
    rc.prefill(dev(k), dev(v), ctx, tq)
    pc.prefill(dev(k), dev(v), ctx, tq)
    for i in range(steps):
        kn = dev(np.stack([k[b, :, ctx[b] + i] for b in range(B)]))
        vn = dev(np.stack([v[b, :, ctx[b] + i] for b in range(B)]))
        q = dev(synth.random_fp16(40 + i, (B, H * r, D)))
        a = host(rc.append_decode(kn, vn, q, SCALE))
        b_ = host(pc.append_decode(kn, vn, q, SCALE))
        assert np.array_equal(a.view(np.uint16), b_.view(np.uint16)), i
    for name in ("k_outliers", "k_codes", "k_scale"):
        g = pc.gather(name)
        ref = host(getattr(rc, name))
        assert np.array_equal(g.view(np.uint32), ref.view(np.uint32)), name


def test_decode_outliers_workload():
    """The batch-8 Llama-2-7B-shaped layer (32 heads, head_dim 128, 4096
    quantized + 128 residual tokens, 2-bit, G = 32) with sporadic key spikes
    and one isolated outlier per key group: prefill bit-exact, every decode
    row within the bar."""
    require_gpu()
    w = synth.WORKLOADS["llama2_7b_b8_ctx4096"].with_(key_spikes=0.01)
    announce("decode outliers llama2_7b_b8_ctx4096 n_out=1")
    k, v = synth.kv(w)
    q = synth.query(w)
    gc = KiviCache(w.batch, w.kv_heads, w.gqa, w.head_dim, w.bits, w.group, w.residual,
                   w.capacity(), outliers=1)
    gc.prefill(dev(k), dev(v), w.tq)
    out = host(gc.decode(dev(q), w.softmax_scale)).astype(np.float64)
    oc = oracle.OracleCache(w.batch, w.kv_heads, w.gqa, w.head_dim, w.bits, w.group,
                            w.residual, w.capacity(), n_out=1)
    oc.prefill(k, v, w.tq)
    assert_cache_equal(gc, oc, what="prefill")
    ref = oc.decode(q, w.softmax_scale)
    err = row_rel_err(out, ref)
    assert err <= ATTN_TOL, err
    torch.cuda.synchronize()

"""GPU decode attention vs the oracle's binary64 output.

Bar: for every (batch, query head) row, max_d |o_gpu - o_ref| / max_d |o_ref|
<= 2e-3 (fp32 accumulation, fp16 inputs and outputs).  Split counts, ragged
tails (a half-filled 64-token value tile, partial residual), empty parts and
GQA ratios are covered; deterministic caches must repeat their output bit for
bit for a fixed split count, the default (shared tiles) within the bar, and
buffers around the output must stay untouched."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_bit_kivi_amd import synth
from kv_cache_bit_kivi_amd.cache import KiviCache
from tests.gpu_util import ATTN_TOL, announce, dev, host, require_gpu, row_rel_err

pytestmark = pytest.mark.gpu


def build_pair(B, H, r, D, bits, G, R, tq, tr, seed, cap=None, k_scale=2.0, v_scale=1.0,
               q_scale=1.0, deterministic=False):
    L = tq + tr
    cap = cap or max(64, (tq + R + 63) // 64 * 64)
    cap = (cap + G - 1) // G * G
    k = synth.random_fp16(seed, (B, H, L, D), scale=k_scale)
    k[..., 5] *= np.float16(10)
    v = synth.random_fp16(seed + 1, (B, H, L, D), scale=v_scale)
    q = synth.random_fp16(seed + 2, (B, H * r, D), scale=q_scale)
    gc = KiviCache(B, H, r, D, bits, G, R, cap, deterministic=deterministic)
    gc.prefill(dev(k), dev(v), tq)
    oc = oracle.OracleCache(B, H, r, D, bits, G, R, cap)
    oc.prefill(k, v, tq)
    return gc, oc, q


SHAPES = [
    # B, H, r, D, bits, G, R, tq, tr
    (1, 1, 1, 128, 2, 32, 32, 512, 0),
    (2, 2, 1, 128, 2, 32, 128, 992, 128),     # half-filled last value tile
    (2, 2, 1, 128, 4, 32, 128, 1024, 77),
    (1, 3, 4, 128, 2, 32, 128, 2016, 100),
    (2, 2, 2, 64, 4, 64, 128, 448, 1),
    (1, 2, 8, 64, 2, 32, 64, 320, 64),
    (3, 1, 1, 32, 2, 32, 32, 96, 31),
    (1, 2, 4, 256, 4, 128, 128, 768, 20),
    (1, 2, 1, 128, 2, 32, 128, 0, 97),        # residual only
    (1, 1, 16, 128, 2, 32, 128, 160, 3),
    (1, 2, 8, 128, 2, 32, 128, 512, 40),       # matrix-core path, r = 8
    (2, 1, 3, 128, 4, 32, 128, 640, 128),      # r = 3 (padded head rows)
    (1, 2, 2, 128, 2, 32, 32, 1984, 32),
    (1, 1, 1, 128, 2, 32, 128, 8192, 5),       # several chunks per wave
    (1, 1, 4, 128, 4, 32, 128, 4096, 128),
    (2, 2, 1, 128, 1, 32, 128, 992, 128),      # 1-bit codes, half-filled last tile
    (1, 3, 4, 128, 1, 32, 64, 2048, 33),
    (2, 2, 1, 128, 3, 32, 128, 1024, 77),      # 3-bit codes
    (1, 2, 8, 128, 3, 32, 128, 512, 40),
    (1, 2, 2, 128, 3, 32, 32, 1984, 32),
    (2, 2, 2, 64, 1, 64, 128, 448, 1),         # generic kernel, 1 bit
    (3, 1, 1, 32, 3, 32, 32, 96, 31),          # generic kernel, 3 bits
]


@pytest.mark.parametrize("shp", SHAPES, ids=lambda s: "B%dH%dr%dD%db%dG%dR%d_tq%d_tr%d" % s)
@pytest.mark.parametrize("splits", [0, 1, 2, 7])
def test_decode_shapes(shp, splits):
    require_gpu()
    B, H, r, D, bits, G, R, tq, tr = shp
    announce(f"decode {shp} splits={splits}")
    gc, oc, q = build_pair(*shp, seed=sum(shp))
    if splits > tq + tr:
        pytest.skip("more splits than tokens")
    ref = oc.decode(q, 0.0883883461356163)
    out = host(gc.decode(dev(q), 0.0883883461356163, num_splits=splits)).astype(np.float64)
    err = row_rel_err(out, ref)
    assert err <= ATTN_TOL, err


@pytest.mark.parametrize("deterministic", [True, False])
def test_decode_deterministic_and_guarded(deterministic):
    """deterministic caches repeat their output bit for bit; with shared
    tiles (the default) repeated outputs stay within the bar of the oracle.
    Neither writes outside the output."""
    require_gpu()
    announce(f"decode determinism / guard band deterministic={deterministic}")
    gc, oc, q = build_pair(2, 4, 2, 128, 2, 32, 128, 1984, 65, seed=5,
                           deterministic=deterministic)
    ref = oc.decode(q, 0.1)
    qd = dev(q)
    n = q.size
    for S in (1, 5):
        buf = torch.full((n + 2048,), 0x7BAD, dtype=torch.int16, device="cuda")
        out = buf[1024:1024 + n].view(torch.float16).view(q.shape)
        for i in range(4):
            gc.decode(qd, 0.1, out=out, num_splits=S)
            b = host(out).copy()
            if i == 0:
                a = b
            elif deterministic:
                assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
            assert row_rel_err(b.astype(np.float64), ref) <= ATTN_TOL
        g = host(buf).view(np.uint16)
        assert np.all(g[:1024] == 0x7BAD) and np.all(g[1024 + n:] == 0x7BAD)


@pytest.mark.parametrize("deterministic", [False, True])
def test_decode_max_splits(deterministic):
    """num_splits at its cap (4096 splits of an 8K context: 32768 waves, most
    without a tile): the wave shares' 32-bit arithmetic at its widest, and the
    combine over 4096 partials, one and four heads."""
    require_gpu()
    for r in (1, 4):
        announce(f"decode max splits r={r} deterministic={deterministic}")
        gc, oc, q = build_pair(1, 1, r, 128, 2, 32, 128, 8128, 100, seed=31 + r,
                               deterministic=deterministic)
        ref = oc.decode(q, 0.0883883461356163)
        out = host(gc.decode(dev(q), 0.0883883461356163, num_splits=4096)).astype(np.float64)
        assert row_rel_err(out, ref) <= ATTN_TOL


def test_split_count_invariance():
    require_gpu()
    announce("split invariance")
    gc, oc, q = build_pair(1, 2, 1, 128, 2, 32, 128, 4064, 128, seed=9)
    gd, _, _ = build_pair(1, 2, 1, 128, 2, 32, 128, 4064, 128, seed=9, deterministic=True)
    qd = dev(q)
    outs = [host(c.decode(qd, 0.09, num_splits=S)).astype(np.float64)
            for c in (gc, gd) for S in (1, 3, 16, 64)]
    for o in outs[1:]:
        assert row_rel_err(o, outs[0]) <= ATTN_TOL


@pytest.mark.parametrize("name,batches", [
    ("single_head_512", None),
    ("llama2_7b_b8_ctx4096", None),
    ("mistral_7b_b32_ctx8192", [0, 17, 31]),
])
def test_decode_workloads(name, batches):
    """Full-size decode of each workload with the automatic split count; the
    oracle computes the listed batch entries (all heads)."""
    require_gpu()
    w = synth.WORKLOADS[name]
    announce(f"decode workload {name}")
    k, v = synth.kv(w)
    q = synth.query(w)
    gc = KiviCache(w.batch, w.kv_heads, w.gqa, w.head_dim, w.bits, w.group, w.residual,
                   w.capacity())
    gc.prefill(dev(k), dev(v), w.tq)
    out = host(gc.decode(dev(q), w.softmax_scale)).astype(np.float64)
    sel = list(range(w.batch)) if batches is None else batches
    oc = oracle.OracleCache(len(sel), w.kv_heads, w.gqa, w.head_dim, w.bits, w.group,
                            w.residual, w.capacity())
    oc.prefill(k[sel], v[sel], w.tq)
    ref = oc.decode(np.ascontiguousarray(q[sel]), w.softmax_scale)
    err = row_rel_err(out[sel], ref)
    assert err <= ATTN_TOL, err


def test_decode_long_context():
    """262,144-token context, batch 1, 32 heads: full-size GPU prefill and
    decode (automatic split-K); the oracle checks heads 0 and 31 (codes and
    attention output)."""
    require_gpu()
    w = synth.WORKLOADS["long_ctx_262144"]
    announce("decode long context 262144")
    gc = KiviCache(w.batch, w.kv_heads, w.gqa, w.head_dim, w.bits, w.group, w.residual,
                   w.capacity())
    # stage K/V head by head to bound host memory
    kd = torch.empty((1, w.kv_heads, w.context, w.head_dim), dtype=torch.float16, device="cuda")
    vd = torch.empty_like(kd)
    for h in range(w.kv_heads):
        kd[0, h] = dev(synth.k_plane(w, 0, h))
        vd[0, h] = dev(synth.v_plane(w, 0, h))
    gc.prefill(kd, vd, w.tq)
    del kd, vd
    q = synth.query(w)
    out = host(gc.decode(dev(q), w.softmax_scale)).astype(np.float64)
    for h in (0, 31):
        k = synth.k_plane(w, 0, h)[None, None]
        v = synth.v_plane(w, 0, h)[None, None]
        oc = oracle.OracleCache(1, 1, 1, w.head_dim, w.bits, w.group, w.residual, w.capacity())
        oc.prefill(k, v, w.tq)
        codes = host(gc.k_codes[0, h])
        assert np.array_equal(codes, oc.k_codes[0, 0])
        assert np.array_equal(host(gc.v_scale[0, h]).view(np.uint32), oc.vs[0, 0].view(np.uint32))
        ref = oc.decode(np.ascontiguousarray(q[:, h:h + 1]), w.softmax_scale)
        err = row_rel_err(out[:, h:h + 1], ref)
        assert err <= ATTN_TOL, (h, err)


@pytest.mark.parametrize("v_scale", [1e-2, 1e-3, 1e3])
@pytest.mark.parametrize("q_scale", [0.25, 3.0])
@pytest.mark.parametrize("bits,r", [(2, 1), (4, 1), (2, 4)])
def test_small_value_scales(v_scale, q_scale, bits, r):
    """Value scales far from 1 (1e-2, 1e-3 and 1e3 times the keys' spread),
    with flat (small q) and sharp (large q) attention: the P.V factor p * s
    spans many binades, and with the lazy softmax reference p reaches 2^8, so
    the factor must keep its relative precision without an fp16 range limit."""
    require_gpu()
    announce(f"decode small values v_scale={v_scale} q_scale={q_scale} bits={bits} r={r}")
    gc, oc, q = build_pair(1, 2, r, 128, bits, 32, 128, 4032, 64, seed=77 + bits + r,
                           v_scale=v_scale, q_scale=q_scale)
    ref = oc.decode(q, 0.0883883461356163)
    out = host(gc.decode(dev(q), 0.0883883461356163)).astype(np.float64)
    err = row_rel_err(out, ref)
    assert err <= ATTN_TOL, err


@pytest.mark.parametrize("meta_half", [False, True])
@pytest.mark.parametrize("r", [1, 2, 4, 8])
def test_decode_large_key_zeros(r, meta_half):
    """Keys around +-3000 (channel offsets), so every key zero is a large
    binary16 value and the zero term carries most of each score: the
    several-heads kernels take the zeros as binary16 matrix operands, one head
    sums them on the vector units; both within the bar of the oracle."""
    require_gpu()
    announce(f"decode large key zeros r={r} meta_half={meta_half}")
    B, H, D, bits, G, R, tq, tr = 2, 2, 128, 2, 32, 128, 1984, 40
    L = tq + tr
    rng_k = synth.random_fp16(71 + r, (B, H, L, D), scale=40.0).astype(np.float32)
    off = np.where(np.arange(D) % 2 == 0, 3000.0, -2500.0).astype(np.float32)
    k = (rng_k + off).astype(np.float16)
    v = synth.random_fp16(72 + r, (B, H, L, D), scale=1.0)
    q = synth.random_fp16(73 + r, (B, H * r, D), scale=0.01)
    cap = (tq + R + 63) // 64 * 64
    gc = KiviCache(B, H, r, D, bits, G, R, cap, meta_half=meta_half)
    gc.prefill(dev(k), dev(v), tq)
    oc = oracle.OracleCache(B, H, r, D, bits, G, R, cap, meta_half=meta_half)
    oc.prefill(k, v, tq)
    ref = oc.decode(q, 0.0883883461356163)
    for S in (0, 3):
        out = host(gc.decode(dev(q), 0.0883883461356163, num_splits=S)).astype(np.float64)
        assert row_rel_err(out, ref) <= ATTN_TOL, (S, row_rel_err(out, ref))

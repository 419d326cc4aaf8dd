"""Ragged batches (a different length for every sequence) on the GPU.

Each sequence of a ragged cache must equal a one-sequence cache holding it
alone: the oracle replays every sequence separately and the GPU's codes,
scales, zeros and residual must match bit for bit, its attention within the
usual row bar.  Covered: ragged prefill (including empty and residual-only
sequences), decode over split counts larger than a short sequence, both
kernel paths, both bit widths, GQA ratios, binary16 metadata, staggered
flushes with the fused step equal to the separate calls, more sequences than
one launch takes, and equal lengths matching the uniform cache exactly (those
comparisons of two calls bit for bit use deterministic caches)."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_bit_kivi_amd import synth
from kv_cache_bit_kivi_amd.cache import KiviCache, RaggedKiviCache
from tests.gpu_util import ATTN_TOL, announce, dev, host, require_gpu, row_rel_err

pytestmark = pytest.mark.gpu

SCALE = 0.0883883461356163
PAIRS = [("k_codes", "k_codes"), ("k_scale", "ks"), ("k_zero", "kz"),
         ("v_codes", "v_codes"), ("v_scale", "vs"), ("v_zero", "vz")]


def bits_of(a):
    return a.view({4: np.uint32, 2: np.uint16}[a.dtype.itemsize])


def assert_seq_equal(gc, b, oc, what=""):
    """Sequence b of the ragged GPU cache equals the one-sequence oracle cache."""
    assert (int(gc.tq[b]), int(gc.tr[b])) == (oc.tq, oc.tr), (what, b)
    for gname, oname in PAIRS:
        g = bits_of(host(getattr(gc, gname)[b:b + 1]))
        o = bits_of(getattr(oc, oname))
        if not np.array_equal(g, o):
            bad = np.argwhere(g != o)
            raise AssertionError(f"{what} seq {b} {gname}: {len(bad)} mismatches at {bad[0]}")
    for gname in ("k_res", "v_res"):
        g = host(getattr(gc, gname)[b:b + 1]).view(np.uint16)[:, :, : oc.tr]
        assert np.array_equal(g, getattr(oc, gname)[:, :, : oc.tr]), (what, b, gname)


def build(B, H, r, D, bits, G, R, ntok, tq, seed, meta_half=False, cap=None):
    T = max(max(ntok), 1)
    cap = cap or max(64, (max(tq) + 2 * R + 63) // 64 * 64)
    cap = (cap + G - 1) // G * G
    k = synth.random_fp16(seed, (B, H, T, D), scale=2.0)
    k[..., 5] *= np.float16(10)
    v = synth.random_fp16(seed + 1, (B, H, T, D))
    gc = RaggedKiviCache(B, H, r, D, bits, G, R, cap, meta_half=meta_half)
    gc.prefill(dev(k), dev(v), ntok, tq)
    ocs = []
    for b in range(B):
        oc = oracle.OracleCache(1, H, r, D, bits, G, R, cap, meta_half=meta_half)
        oc.prefill(k[b:b + 1, :, : ntok[b]], v[b:b + 1, :, : ntok[b]], tq[b])
        ocs.append(oc)
    return gc, ocs, k, v


def check_decode(gc, ocs, q, out, what):
    for b, oc in enumerate(ocs):
        ref = oc.decode(np.ascontiguousarray(q[b:b + 1]), SCALE)
        err = row_rel_err(out[b:b + 1].astype(np.float64), ref)
        assert err <= ATTN_TOL, (what, b, err)


CASES = [
    # B, H, r, D, bits, G, R, ntok, tq, meta_half
    (4, 2, 1, 128, 2, 32, 128, [69, 1152, 320, 2125], [64, 1024, 320, 2048], False),
    (4, 2, 1, 128, 2, 32, 128, [3, 1152, 97, 736], [0, 1024, 0, 640], True),
    (3, 2, 4, 128, 4, 32, 64, [100, 700, 1500], [64, 640, 1472], False),
    (3, 1, 8, 128, 2, 32, 128, [40, 992, 2100], [0, 960, 1984], False),
    (2, 3, 2, 128, 4, 32, 32, [64, 2000], [64, 1984], True),
    (3, 2, 2, 64, 2, 32, 32, [60, 300, 2], [32, 288, 0], False),       # generic kernel
    (2, 2, 1, 32, 4, 32, 32, [31, 450], [0, 448], True),              # generic kernel
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dr%dD%db%dG%dR%d" % c[:7] + (
    "_m16" if c[9] else ""))
@pytest.mark.parametrize("splits", [0, 1, 5])
def test_ragged_prefill_decode(case, splits):
    require_gpu()
    B, H, r, D, bits, G, R, ntok, tq, mh = case
    announce(f"ragged prefill+decode {case} splits={splits}")
    gc, ocs, _, _ = build(B, H, r, D, bits, G, R, ntok, tq, seed=sum(ntok) + bits, meta_half=mh)
    for b, oc in enumerate(ocs):
        assert_seq_equal(gc, b, oc, "prefill")
    q = synth.random_fp16(7 + B, (B, H * r, D))
    out = host(gc.decode(dev(q), SCALE, num_splits=splits))
    check_decode(gc, ocs, q, out, f"decode S={splits}")
    # shared tiles: a second call may group the sums differently, within the bar
    again = host(gc.decode(dev(q), SCALE, num_splits=splits))
    check_decode(gc, ocs, q, again, f"decode again S={splits}")


@pytest.mark.parametrize("bits,meta_half,r", [(2, False, 1), (4, True, 2), (2, False, 4)])
def test_ragged_stream_fused(bits, meta_half, r):
    """Staggered residual fill levels, so the sequences flush at different
    steps (and one starts empty): the fused step equals append + decode bit
    for bit, each sequence equals its oracle replay."""
    require_gpu()
    announce(f"ragged stream bits={bits} mh={meta_half} r={r}")
    B, H, D, G, R = 4, 2, 128, 32, 32
    tq = [64, 128, 0, 32]
    tr0 = [R, R - 3, 5, 0]
    ntok = [a + b for a, b in zip(tq, tr0)]
    steps = R + 6
    cap = (max(tq) + R * 3 + 63) // 64 * 64
    T = max(ntok) + steps
    k = synth.random_fp16(300 + bits, (B, H, T, D), scale=1.5)
    k[..., 2] *= np.float16(10)
    v = synth.random_fp16(310 + bits, (B, H, T, D))
    qs = synth.random_fp16(320 + bits, (steps, B, H * r, D))
    sep = RaggedKiviCache(B, H, r, D, bits, G, R, cap, meta_half=meta_half, deterministic=True)
    fus = RaggedKiviCache(B, H, r, D, bits, G, R, cap, meta_half=meta_half, deterministic=True)
    kd, vd = dev(k), dev(v)
    sep.prefill(kd, vd, ntok, tq)
    fus.prefill(kd, vd, ntok, tq)
    ocs = []
    for b in range(B):
        oc = oracle.OracleCache(1, H, r, D, bits, G, R, cap, meta_half=meta_half)
        oc.prefill(k[b:b + 1, :, : ntok[b]], v[b:b + 1, :, : ntok[b]], tq[b])
        ocs.append(oc)
    for i in range(steps):
        # the new token of sequence b is its token ntok[b] + i
        kn = np.stack([k[b, :, ntok[b] + i] for b in range(B)])
        vn = np.stack([v[b, :, ntok[b] + i] for b in range(B)])
        q = dev(qs[i])
        sep.append(dev(kn), dev(vn))
        o_sep = host(sep.decode(q, SCALE))
        o_fus = host(fus.append_decode(dev(kn), dev(vn), q, SCALE))
        assert np.array_equal(o_fus.view(np.uint16), o_sep.view(np.uint16)), f"step {i}"
        assert np.array_equal(fus.tq, sep.tq) and np.array_equal(fus.tr, sep.tr)
        for b, oc in enumerate(ocs):
            oc.append(np.ascontiguousarray(kn[b:b + 1]), np.ascontiguousarray(vn[b:b + 1]))
        if i in (0, 1, 3, R - 1, R + 5):
            for b, oc in enumerate(ocs):
                assert_seq_equal(fus, b, oc, f"fused step {i}")
                assert_seq_equal(sep, b, oc, f"separate step {i}")
        check_decode(fus, ocs, qs[i], o_fus, f"step {i}")
    assert [oc.flushes for oc in ocs] == [2, 2, 1, 1]


def test_ragged_many_sequences():
    """130 sequences: more than one launch's worth, with the split-K
    workspace carved per launch."""
    require_gpu()
    announce("ragged 130 sequences")
    B, H, r, D, bits, G, R = 130, 1, 2, 128, 2, 32, 32
    rng = np.random.default_rng(5)
    tq = (rng.integers(0, 12, B) * 32).tolist()
    ntok = [t + int(rng.integers(1, R + 1)) for t in tq]
    gc, ocs, k, v = build(B, H, r, D, bits, G, R, ntok, tq, seed=41)
    for b in (0, 64, 127, 128, 129):
        assert_seq_equal(gc, b, ocs[b], "prefill")
    q = synth.random_fp16(43, (B, H * r, D))
    for S in (1, 3):
        out = host(gc.decode(dev(q), SCALE, num_splits=S))
        check_decode(gc, ocs, q, out, f"S={S}")
    kn = synth.random_fp16(44, (B, H, D))
    vn = synth.random_fp16(45, (B, H, D))
    out = host(gc.append_decode(dev(kn), dev(vn), dev(q), SCALE))
    for b, oc in enumerate(ocs):
        oc.append(np.ascontiguousarray(kn[b:b + 1]), np.ascontiguousarray(vn[b:b + 1]))
    for b in (0, 127, 128, 129):
        assert_seq_equal(gc, b, ocs[b], "append")
    check_decode(gc, ocs, q, out, "fused")


@pytest.mark.parametrize("D,r,S", [(128, 1, 0), (128, 4, 3), (64, 2, 2)])
def test_ragged_equal_lengths_match_uniform(D, r, S):
    """With every sequence at the same lengths, the ragged calls reproduce the
    uniform cache's output bit for bit (same kernels, lengths per launch)."""
    require_gpu()
    announce(f"ragged == uniform D={D} r={r} S={S}")
    B, H, bits, G, R = 3, 2, 2, 32, 128
    tq, tr = 1024, 77
    cap = 1280
    k = synth.random_fp16(61, (B, H, tq + tr, D), scale=2.0)
    v = synth.random_fp16(62, (B, H, tq + tr, D))
    q = dev(synth.random_fp16(63, (B, H * r, D)))
    uc = KiviCache(B, H, r, D, bits, G, R, cap, deterministic=True)
    rc = RaggedKiviCache(B, H, r, D, bits, G, R, cap, deterministic=True)
    kd, vd = dev(k), dev(v)
    uc.prefill(kd, vd, tq)
    rc.prefill(kd, vd, [tq + tr] * B, [tq] * B)
    a = host(uc.decode(q, SCALE, num_splits=S))
    b = host(rc.decode(q, SCALE, num_splits=S))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    kn, vn = dev(synth.random_fp16(64, (B, H, D))), dev(synth.random_fp16(65, (B, H, D)))
    a = host(uc.append_decode(kn, vn, q, SCALE, num_splits=S))
    b = host(rc.append_decode(kn, vn, q, SCALE, num_splits=S))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    torch.cuda.synchronize()

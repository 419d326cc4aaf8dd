"""Paged quantized store on the GPU: the same calls on a paged cache and on a
ragged (contiguous) cache give bit-identical outputs at every step, and the
pages, gathered through the block table, equal the contiguous buffers bit for
bit (through prefill, staggered flushes and fused steps).  The table is a
shuffled page order with spare pages that must stay untouched and, in one
case, -1 entries past every sequence's reach that must never be needed.  The
ragged cache itself is checked against the oracle in test_gpu_ragged.py, and
the paged store is also checked against the oracle directly (gathered codes,
scales, zeros and outlier words bit for bit, attention within the row bar)
for every code width, both metadata widths, both kernel paths, key outliers
and pre-RoPE keys.  The caches compared bit for bit are deterministic ones."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_bit_kivi_amd import synth
from kv_cache_bit_kivi_amd.cache import PagedKiviCache, RaggedKiviCache
from tests.gpu_util import ATTN_TOL, announce, dev, host, require_gpu, row_rel_err

pytestmark = pytest.mark.gpu

SCALE = 0.0883883461356163
QUANT = ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero")


def bits_of(a):
    return a.view({4: np.uint32, 2: np.uint16}[a.dtype.itemsize])


def assert_same_cache(pc, rc, what):
    assert np.array_equal(pc.tq, rc.tq) and np.array_equal(pc.tr, rc.tr), what
    for name in QUANT:
        g = bits_of(pc.gather(name))
        r = bits_of(host(getattr(rc, name)))
        if not np.array_equal(g, r):
            bad = np.argwhere(g != r)
            raise AssertionError(f"{what} {name}: {len(bad)} mismatches, first at {bad[0]}")
    for name in ("k_res", "v_res"):
        assert np.array_equal(host(getattr(pc, name)).view(np.uint16),
                              host(getattr(rc, name)).view(np.uint16)), (what, name)


def run_pair(B, H, r, D, bits, G, R, P, ctx, steps, seed, meta_half=False, splits=0,
             trim_table=False):
    tq = [c - ((c - 1) % R + 1) if c > 0 else 0 for c in ctx]
    T = max(ctx) + steps
    cap = ((max(tq) + (steps // R + 2) * R + P - 1) // P) * P
    mp = cap // P
    spare = 5
    rng = np.random.default_rng(seed)
    table = rng.permutation(B * mp + spare)[: B * mp].astype(np.int32).reshape(B, mp)
    if trim_table:
        # logical pages past what each sequence can reach in this run: -1
        for b in range(B):
            need = (tq[b] + (steps // R + 1) * R + P - 1) // P
            table[b, need:] = -1
    used = set(int(x) for x in table.ravel() if x >= 0)
    spare_pages = [p for p in range(B * mp + spare) if p not in used]
    k = synth.random_fp16(seed, (B, H, T, D), scale=2.0)
    k[..., 3] *= np.float16(10)
    v = synth.random_fp16(seed + 1, (B, H, T, D))
    qs = synth.random_fp16(seed + 2, (steps + 1, B, H * r, D))
    rc = RaggedKiviCache(B, H, r, D, bits, G, R, cap, meta_half=meta_half, deterministic=True)
    pc = PagedKiviCache(B, H, r, D, bits, G, R, cap, P, num_pages=B * mp + spare, table=table,
                        meta_half=meta_half, deterministic=True)
    kd, vd = dev(k), dev(v)
    rc.prefill(kd, vd, ctx, tq)
    pc.prefill(kd, vd, ctx, tq)
    assert_same_cache(pc, rc, "prefill")
    q = dev(qs[0])
    a = host(rc.decode(q, SCALE, num_splits=splits))
    b = host(pc.decode(q, SCALE, num_splits=splits))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), "decode"
    for i in range(steps):
        kn = dev(np.stack([k[bb, :, ctx[bb] + i] for bb in range(B)]))
        vn = dev(np.stack([v[bb, :, ctx[bb] + i] for bb in range(B)]))
        q = dev(qs[i + 1])
        a = host(rc.append_decode(kn, vn, q, SCALE, num_splits=splits))
        b = host(pc.append_decode(kn, vn, q, SCALE, num_splits=splits))
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), f"step {i}"
    assert_same_cache(pc, rc, "after steps")
    for name in QUANT:   # spare pages never written
        pool = host(getattr(pc, name))
        for p in spare_pages:
            assert not np.any(bits_of(pool[p])), (name, p)
    return pc, rc, k, v, tq


CASES = [
    # B, H, r, D, bits, G, R, P, ctx, meta_half
    (4, 2, 1, 128, 2, 32, 32, 128, [69, 400, 1, 255], False),
    (3, 2, 4, 128, 4, 32, 64, 256, [100, 700, 64], False),
    (2, 1, 8, 128, 2, 32, 32, 64, [300, 97], True),
    (3, 2, 2, 64, 2, 32, 32, 64, [60, 300, 2], False),      # generic kernel
    (2, 2, 1, 32, 4, 32, 32, 64, [31, 450], True),          # generic kernel
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dr%dD%db%dG%dR%dP%d" % c[:8] + (
    "_m16" if c[9] else ""))
@pytest.mark.parametrize("splits", [0, 3])
def test_paged_equals_ragged(case, splits):
    require_gpu()
    B, H, r, D, bits, G, R, P, ctx, mh = case
    announce(f"paged == ragged {case} splits={splits}")
    run_pair(B, H, r, D, bits, G, R, P, ctx, steps=R + 5, seed=sum(ctx) + P, meta_half=mh,
             splits=splits)


def test_paged_trimmed_table_and_oracle():
    """Table entries past every sequence's reach are -1 (never looked up);
    the paged output also meets the oracle directly."""
    require_gpu()
    announce("paged trimmed table + oracle")
    B, H, r, D, bits, G, R, P = 3, 2, 2, 128, 2, 32, 32, 64
    ctx = [200, 40, 129]
    steps = R + 3
    pc, rc, k, v, tq = run_pair(B, H, r, D, bits, G, R, P, ctx, steps, seed=77,
                                trim_table=True)
    q = synth.random_fp16(78, (B, H * r, D))
    out = host(pc.decode(dev(q), SCALE))
    for b in range(B):
        L = ctx[b] + steps
        oc = oracle.OracleCache(1, H, r, D, bits, G, R, pc.shape.capacity)
        # the same token sequence, streamed into a one-sequence oracle cache
        oc.prefill(k[b:b + 1, :, : ctx[b]], v[b:b + 1, :, : ctx[b]], tq[b])
        for i in range(steps):
            oc.append(np.ascontiguousarray(k[b:b + 1, :, ctx[b] + i]),
                      np.ascontiguousarray(v[b:b + 1, :, ctx[b] + i]))
        assert oc.tq + oc.tr == L
        ref = oc.decode(np.ascontiguousarray(q[b:b + 1]), SCALE)
        assert row_rel_err(out[b:b + 1].astype(np.float64), ref) <= ATTN_TOL, b


def test_paged_many_sequences():
    """130 sequences: the block-table rows are offset per launch."""
    require_gpu()
    announce("paged 130 sequences")
    rng = np.random.default_rng(9)
    ctx = rng.integers(1, 400, 130).tolist()
    run_pair(130, 1, 1, 128, 2, 32, 32, 64, ctx, steps=3, seed=10, splits=2)
    torch.cuda.synchronize()


ORACLE_CASES = [
    # B, H, r, D, bits, G, R, P, ctx, meta_half, outliers, rope_theta
    (3, 2, 1, 128, 4, 32, 32, 64, [69, 300, 130], False, 0, 0.0),
    (3, 2, 2, 128, 2, 32, 32, 128, [200, 33, 257], True, 0, 0.0),
    (2, 2, 4, 128, 3, 32, 64, 64, [150, 390], True, 0, 0.0),
    (2, 1, 8, 128, 1, 32, 32, 64, [100, 260], False, 0, 0.0),
    (3, 2, 1, 64, 2, 32, 32, 64, [60, 300, 2], False, 0, 0.0),        # generic kernel
    (3, 2, 1, 128, 2, 32, 32, 128, [140, 300, 40], False, 1, 0.0),    # outliers, matrix cores
    (2, 2, 2, 128, 4, 32, 32, 64, [90, 280], True, 2, 0.0),           # outliers, matrix cores
    (2, 2, 2, 64, 4, 32, 32, 64, [70, 200], False, 3, 0.0),           # outliers, generic
    (3, 2, 1, 128, 2, 32, 32, 64, [100, 330, 64], False, 0, 10000.0),  # pre-RoPE keys
]


@pytest.mark.parametrize("case", ORACLE_CASES, ids=lambda c: "B%dH%dr%dD%db%dG%dR%dP%d" % c[:8] + (
    "_m16" if c[9] else "") + (f"_o{c[10]}" if c[10] else "") + ("_rope" if c[11] else ""))
def test_paged_vs_oracle(case):
    """The paged store against the oracle directly, sequence by sequence:
    after a prefill and R + 5 fused steps (every sequence flushes once), the
    pages gathered through a shuffled block table equal a one-sequence
    oracle cache's codes, scales, zeros and key-outlier words bit for bit,
    the residuals equal its residual, and the attention of the prefill, of a
    step in the middle and of the last step meets its attention within the
    row bar."""
    require_gpu()
    B, H, r, D, bits, G, R, P, ctx, mh, n_out, theta = case
    announce(f"paged vs oracle {case}")
    steps = R + 5
    tq = [c - ((c - 1) % R + 1) if c > 0 else 0 for c in ctx]
    T = max(ctx) + steps
    cap = ((max(tq) + (steps // R + 2) * R + P - 1) // P) * P
    mp = cap // P
    rng = np.random.default_rng(sum(ctx) + bits)
    table = rng.permutation(B * mp + 3)[: B * mp].astype(np.int32).reshape(B, mp)
    seed = 300 + sum(ctx) + bits
    k = (synth.spiky_fp16(seed, (B, H, T, D), rate=0.03, scale=2.0) if n_out
         else synth.random_fp16(seed, (B, H, T, D), scale=2.0))
    k[..., 3] *= np.float16(8)
    v = synth.random_fp16(seed + 1, (B, H, T, D))
    qs = synth.random_fp16(seed + 2, (steps + 1, B, H * r, D))
    pc = PagedKiviCache(B, H, r, D, bits, G, R, cap, P, num_pages=B * mp + 3, table=table,
                        meta_half=mh, outliers=n_out, rope_theta=theta)
    pc.prefill(dev(k), dev(v), ctx, tq)
    ocs = []
    for b in range(B):
        oc = oracle.OracleCache(1, H, r, D, bits, G, R, cap, meta_half=mh, n_out=n_out,
                                rope_theta=theta)
        oc.prefill(k[b:b + 1, :, : ctx[b]], v[b:b + 1, :, : ctx[b]], tq[b])
        ocs.append(oc)

    def check_attn(out, q, what):
        got = host(out).astype(np.float64)
        for b in range(B):
            ref = ocs[b].decode(np.ascontiguousarray(q[b:b + 1]), SCALE)
            err = row_rel_err(got[b:b + 1], ref)
            assert err <= ATTN_TOL, (what, b, err)

    check_attn(pc.decode(dev(qs[0]), SCALE), qs[0], "prefill")
    for i in range(steps):
        kn = np.stack([k[b, :, ctx[b] + i] for b in range(B)])
        vn = np.stack([v[b, :, ctx[b] + i] for b in range(B)])
        out = pc.append_decode(dev(kn), dev(vn), dev(qs[i + 1]), SCALE)
        for b in range(B):
            ocs[b].append(np.ascontiguousarray(kn[b:b + 1]), np.ascontiguousarray(vn[b:b + 1]))
        if i in (R // 2, steps - 1):
            check_attn(out, qs[i + 1], f"step {i}")
    assert all(oc.flushes >= 1 for oc in ocs)
    assert np.array_equal(pc.tq, [oc.tq for oc in ocs])
    assert np.array_equal(pc.tr, [oc.tr for oc in ocs])
    pairs = [("k_codes", "k_codes"), ("k_scale", "ks"), ("k_zero", "kz"),
             ("v_codes", "v_codes"), ("v_scale", "vs"), ("v_zero", "vz")]
    if n_out:
        pairs.append(("k_outliers", "k_outl"))
    for gname, oname in pairs:
        g = bits_of(pc.gather(gname))
        for b in range(B):
            o = bits_of(getattr(ocs[b], oname)[0])
            if not np.array_equal(g[b], o):
                bad = np.argwhere(g[b] != o)
                raise AssertionError(f"{gname} seq {b}: {len(bad)} mismatches, first at "
                                     f"{bad[0].tolist()}")
    kr = host(pc.k_res).view(np.uint16)
    vr = host(pc.v_res).view(np.uint16)
    for b in range(B):
        t = ocs[b].tr
        assert np.array_equal(kr[b, :, :t], ocs[b].k_res[0, :, :t]), b
        assert np.array_equal(vr[b, :, :t], ocs[b].v_res[0, :, :t]), b

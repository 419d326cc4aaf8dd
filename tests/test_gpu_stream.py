"""GPU streaming append / flush vs the oracle, bit-exact on every buffer, and
the decode attention of the streamed caches within the row bar."""
import numpy as np
import pytest

import oracle
from kv_cache_bit_kivi_amd import synth
from kv_cache_bit_kivi_amd.cache import KiviCache
from tests.gpu_util import (ATTN_TOL, announce, assert_cache_equal, dev, host, require_gpu,
                            row_rel_err)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("G,R,D", [(32, 32, 64), (32, 128, 128), (64, 128, 128), (128, 128, 256)])
def test_append_stream_small(bits, G, R, D):
    require_gpu()
    announce(f"append stream bits={bits} G={G} R={R} D={D}")
    B, H = 2, 3
    tq0, tr0, n = G * 2, R, 2 * R + 7
    T = tq0 + tr0 + n
    k = synth.random_fp16(60 + bits + G, (B, H, T, D), scale=1.5)
    v = synth.random_fp16(70 + bits + G, (B, H, T, D))
    k[..., 2] *= np.float16(10)
    cap = (T + R + 63) // 64 * 64
    cap = (cap + G - 1) // G * G
    gc = KiviCache(B, H, 1, D, bits, G, R, cap)
    oc = oracle.OracleCache(B, H, 1, D, bits, G, R, cap)
    gc.prefill(dev(k[:, :, : tq0 + tr0]), dev(v[:, :, : tq0 + tr0]), tq0)
    oc.prefill(k[:, :, : tq0 + tr0], v[:, :, : tq0 + tr0], tq0)
    assert_cache_equal(gc, oc, what="prefill")
    for i in range(n):
        t = tq0 + tr0 + i
        kn, vn = np.ascontiguousarray(k[:, :, t]), np.ascontiguousarray(v[:, :, t])
        gc.append(dev(kn), dev(vn))
        oc.append(kn, vn)
        if i in (0, 1, R - 1, R, n - 1):
            assert_cache_equal(gc, oc, what=f"step {i}")
    assert oc.flushes >= 2


@pytest.mark.parametrize("name", ["stream_b64_4bit", "stream_b64_2bit"])
def test_streaming_workload(name):
    """The streaming workload at full size (batch 64, 32 heads, prefill 4096,
    256 appended tokens, two flushes); the oracle replays batch entries 0 and
    41 and every buffer must match bit for bit."""
    require_gpu()
    w = synth.WORKLOADS[name]
    announce(f"streaming workload {name}")
    sel = [0, 41]
    k, v = synth.kv(w)
    cap = w.capacity(w.steps)
    gc = KiviCache(w.batch, w.kv_heads, w.gqa, w.head_dim, w.bits, w.group, w.residual, cap)
    gc.prefill(dev(k), dev(v), w.tq)
    oc = oracle.OracleCache(len(sel), w.kv_heads, w.gqa, w.head_dim, w.bits, w.group,
                            w.residual, cap)
    oc.prefill(k[sel], v[sel], w.tq)
    del k, v
    for s in range(1, w.steps + 1):
        kn, vn = synth.new_token(w, s)
        gc.append(dev(kn), dev(vn))
        oc.append(np.ascontiguousarray(kn[sel]), np.ascontiguousarray(vn[sel]))
        if s in (1, 2, 128, 129, 130, 256):
            assert_cache_equal(gc, oc, planes=sel, what=f"{name} step {s}")
    assert oc.flushes == 2


@pytest.mark.parametrize("name", ["stream_b64_4bit", "stream_b64_2bit"])
def test_streaming_workload_attention(name):
    """The step the benchmark times, at full size: every one of the 256 steps
    appends and decodes (kivi_append_decode_attn, except steps 2 and 129,
    which take kivi_append then kivi_decode_attn, so both routes meet a flush
    at full size).  At steps 1, 2, 128, 129, 130 and 256 the attention of
    batch entries 0 and 41 meets the oracle's within the row bar and every
    buffer of those entries equals the oracle's bit for bit."""
    require_gpu()
    w = synth.WORKLOADS[name]
    announce(f"streaming workload attention {name}")
    sel = [0, 41]
    k, v = synth.kv(w)
    cap = w.capacity(w.steps)
    gc = KiviCache(w.batch, w.kv_heads, w.gqa, w.head_dim, w.bits, w.group, w.residual, cap)
    gc.prefill(dev(k), dev(v), w.tq)
    oc = oracle.OracleCache(len(sel), w.kv_heads, w.gqa, w.head_dim, w.bits, w.group,
                            w.residual, cap)
    oc.prefill(k[sel], v[sel], w.tq)
    del k, v
    worst = 0.0
    for s in range(1, w.steps + 1):
        kn, vn = synth.new_token(w, s)
        q = synth.query(w, s)
        if s in (2, 129):
            gc.append(dev(kn), dev(vn))
            out = gc.decode(dev(q), w.softmax_scale)
        else:
            out = gc.append_decode(dev(kn), dev(vn), dev(q), w.softmax_scale)
        oc.append(np.ascontiguousarray(kn[sel]), np.ascontiguousarray(vn[sel]))
        if s in (1, 2, 128, 129, 130, 256):
            got = host(out)[sel].astype(np.float64)
            ref = oc.decode(np.ascontiguousarray(q[sel]), w.softmax_scale)
            err = row_rel_err(got, ref)
            worst = max(worst, err)
            assert err <= ATTN_TOL, (name, s, err)
            assert_cache_equal(gc, oc, planes=sel, what=f"{name} step {s}")
    assert oc.flushes == 2
    print(f"{name}: worst row error {worst:.2e}")

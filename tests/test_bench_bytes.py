"""The benchmark's algorithmic byte counts agree with the library's own
buffer sizes (kivi_cache_bytes) for a cache filled to capacity, for both
metadata widths, so the roofline's bytes per launch are the cache's bytes."""
import ctypes

import numpy as np

import pytest

import bench
from kv_cache_bit_kivi_amd import _lib
from kv_cache_bit_kivi_amd.cache import make_shape


@pytest.mark.parametrize("meta_half", [False, True])
@pytest.mark.parametrize("B,H,r,D,bits,G,R,cap", [
    (8, 32, 1, 128, 2, 32, 128, 4096),
    (2, 8, 4, 128, 4, 32, 128, 1024),
    (1, 2, 2, 64, 2, 64, 64, 512),
])
def test_decode_bytes_match_cache_sizes(meta_half, B, H, r, D, bits, G, R, cap):
    s = make_shape(B, H, r, D, bits, G, R, cap, meta_half)
    sz = [ctypes.c_size_t() for _ in range(6)]
    assert _lib.kivi_cache_bytes(ctypes.byref(s), *[ctypes.byref(x) for x in sz]) == 0
    kc, km, vc, vm, res, q = [x.value for x in sz]
    mb = 2 if meta_half else 4
    # decode at tq = cap, tr = R: every code, 2 metadata arrays each side,
    # both residual planes, the query and the output
    want = kc + vc + 2 * km + 2 * vm + 2 * res + 2 * q
    assert bench.decode_bytes(B, H, r, D, bits, G, cap, R, mb) == want
    # a flush reads R tokens of K and V and writes their codes and metadata;
    # plus the new token read and written
    per_tok_codes = kc // cap
    flush = (2 * res + 2 * per_tok_codes * R + 2 * (km // (cap // G)) * (R // G)
             + 2 * (vm // cap) * R)
    tok = 2 * B * H * D * 2 * 2
    assert bench.append_bytes(B, H, D, bits, G, R, True, mb) == tok + flush
    assert bench.append_bytes(B, H, D, bits, G, R, False, mb) == tok


@pytest.mark.parametrize("n_out", [1, 2])
def test_outlier_bytes_match_store_size(n_out):
    """With key outliers, a decode over a full cache also reads the whole
    outlier store, and a flush writes R/G groups of it."""
    B, H, r, D, bits, G, R, cap = 8, 32, 1, 128, 2, 32, 128, 4096
    s = make_shape(B, H, r, D, bits, G, R, cap, False, n_out)
    nb = ctypes.c_size_t()
    assert _lib.kivi_outlier_bytes(ctypes.byref(s), 0, 0, ctypes.byref(nb)) == 0
    base = bench.decode_bytes(B, H, r, D, bits, G, cap, R, 4)
    assert bench.decode_bytes(B, H, r, D, bits, G, cap, R, 4, n_out) == base + nb.value
    f0 = bench.append_bytes(B, H, D, bits, G, R, True, 4)
    assert bench.append_bytes(B, H, D, bits, G, R, True, 4, n_out) == f0 + nb.value * R // cap


@pytest.mark.parametrize("meta_half", [False, True])
def test_cpu_baseline_runs_its_sample(meta_half):
    """The CPU leg keeps stepping until its time budget (or step cap) is
    reached, for both metadata widths."""
    from kv_cache_bit_kivi_amd import synth
    w = synth.WORKLOADS["single_head_512"]
    r = bench.cpu_baseline(w, min_seconds=0.05, max_seconds=5.0, meta_half=meta_half,
                           workers=1)
    steps = int(r["sample"].split()[0])
    assert steps > 1 and r["one_core"]["steps"] == steps
    r = bench.cpu_baseline(w.with_(key_spikes=0.01), min_seconds=0.05, max_seconds=5.0,
                           meta_half=meta_half, n_out=2, workers=1)
    assert int(r["sample"].split()[0]) > 1
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["value"] > 0
    assert r["cpu_model"] and r["host_cores_visible"] >= 1


def test_ragged_workload_lengths():
    """The ragged workload's per-sequence lengths: inside [min_context,
    context], seeded (stable), tq a multiple of the group, 1..R residual."""
    from kv_cache_bit_kivi_amd import synth
    w = synth.WORKLOADS["ragged_b16_ctx512_8192"]
    ctx, tq = w.contexts(), w.tqs()
    assert len(ctx) == w.batch and w.ragged
    assert ctx.min() >= w.min_context and ctx.max() <= w.context
    assert len(set(ctx.tolist())) > w.batch // 2          # genuinely ragged
    assert np.all(tq % w.group == 0)
    assert np.all((ctx - tq >= 1) & (ctx - tq <= w.residual))
    assert np.array_equal(ctx, w.contexts())
    u = synth.WORKLOADS["llama2_7b_b8_ctx4096"]
    assert not u.ragged and np.all(u.contexts() == u.context) and np.all(u.tqs() == u.tq)


def test_cpu_baseline_ragged_sample():
    from kv_cache_bit_kivi_amd import synth
    w = synth.WORKLOADS["ragged_b16_ctx512_8192"].with_(batch=3, q_heads=2, kv_heads=2,
                                                        context=384, min_context=40)
    r = bench.cpu_baseline(w, min_seconds=0.05, max_seconds=5.0, workers=1)
    assert int(r["sample"].split()[0]) > 1 and r["value"] > 0


def test_cpu_baseline_multi_core():
    """The multi-core leg fans the (batch, KV-head) units over worker
    processes and moves the same bytes per step as one core does."""
    from kv_cache_bit_kivi_amd import synth
    w = synth.WORKLOADS["single_head_512"].with_(batch=2, q_heads=4, kv_heads=2, context=256,
                                                 tq=224)
    r = bench.cpu_baseline(w, min_seconds=0.05, max_seconds=5.0, workers=3)
    assert r["cores"] == 3 and r["value"] > 0 and r["one_core"]["value"] > 0
    assert "over 3 processes" in r["sample"]


def test_window_bytes():
    """With the value window, the tokens [L - R, tq) have quantized keys and
    fp16 values: the decode reads 2 D value bytes each instead of their
    codes, scales and zeros; everything else is unchanged.  The append adds
    the leaving value, and its flush covers the keys only."""
    B, H, r, D, bits, G, R = 2, 4, 1, 128, 2, 32, 128
    for mb in (4, 2):
        for tq, tr in ((3968, 127), (4096, 1), (0, 60), (64, 100)):
            tv = max(0, tq + tr - R)
            diff = int(bench.decode_bytes(B, H, r, D, bits, G, tq, tr, mb, 0, True, R)) - \
                bench.decode_bytes(B, H, r, D, bits, G, tq, tr, mb)
            assert diff == B * H * (tq - tv) * (2 * D - D * bits // 8 - (D // G) * 2 * mb)
        base = bench.append_bytes(B, H, D, bits, G, R, False, mb)
        leave = bench.append_bytes(B, H, D, bits, G, R, False, mb, 0, True, True)
        assert leave - base == B * H * (2 * D + D * bits // 8 + (D // G) * 2 * mb)
        full = bench.append_bytes(B, H, D, bits, G, R, True, mb)
        keys = bench.append_bytes(B, H, D, bits, G, R, True, mb, 0, True, False)
        assert full - keys == B * H * (R * D * 2 + R * D * bits // 8 + R * (D // G) * 2 * mb)
    # prefill: the window keeps the R newest values, so max(0, T - R) are quantized
    assert bench.prefill_bytes(H, D, bits, G, 3968, 128, 4, 0, True, R) == \
        bench.prefill_bytes(H, D, bits, G, 3968, 128, 4)
    assert bench.prefill_bytes(H, D, bits, G, 64, 100, 4, 0, True, R) < \
        bench.prefill_bytes(H, D, bits, G, 64, 100, 4) + H * 64 * D * 4

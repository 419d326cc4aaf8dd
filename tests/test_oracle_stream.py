"""Pins of the oracle's streaming append / flush.

Pages: study.space summary of KIVI -- the cache is split into grouped
(quantized) and residual (full-precision) parts, new tokens are appended along
the token axis, key groups span tokens; scholarfeed "KIVI" quote page -- a
fixed-length residual buffer of recent unquantized key/value pairs.
Reading: a token arriving at a full residual (R tokens) first flushes all R
into the quantized part.
"""
import numpy as np
import pytest

import oracle
from kv_cache_bit_kivi_amd import synth
from tests.helpers import unpack_k, unpack_v


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("G,R", [(32, 32), (32, 128), (64, 128)])
def test_stream_equals_one_shot(oracle_lib, bits, G, R):
    """prefill + n appends leaves exactly the codes/scales/zeros that one
    quantization of the same tokens gives, and the newest tokens in the
    residual."""
    B, H, D = 2, 2, 64
    tq0, tr0, n = 2 * G, R, 3 * R + 5
    T = tq0 + tr0 + n
    k = synth.random_fp16(40 + bits, (B, H, T, D), scale=1.5)
    v = synth.random_fp16(50 + bits, (B, H, T, D))
    cap = ((T + R) // 64 + 1) * 64
    c = oracle.OracleCache(B, H, 1, D, bits, G, R, cap)
    c.prefill(k[:, :, : tq0 + tr0], v[:, :, : tq0 + tr0], tq0)
    for i in range(n):
        t = tq0 + tr0 + i
        c.append(k[:, :, t], v[:, :, t])
        assert 1 <= c.tr <= R and c.tq % G == 0 and c.tq + c.tr == t + 1
    assert c.flushes == (tr0 + n - 1) // R
    tq = c.tq
    ck, sk, zk = oracle.quantize_k(k, bits, G, cap, ntok=tq)
    cv, sv, zv = oracle.quantize_v(v, bits, G, cap, ntok=tq)
    assert np.array_equal(unpack_k(c.k_codes, bits, tq, D), unpack_k(ck, bits, tq, D))
    assert np.array_equal(unpack_v(c.v_codes, bits, tq, D), unpack_v(cv, bits, tq, D))
    assert np.array_equal(c.ks[:, :, : tq // G], sk[:, :, : tq // G])
    assert np.array_equal(c.kz[:, :, : tq // G], zk[:, :, : tq // G])
    assert np.array_equal(c.vs[:, :, :tq], sv[:, :, :tq])
    assert np.array_equal(c.vz[:, :, :tq], zv[:, :, :tq])
    assert np.array_equal(c.k_res[:, :, : c.tr], k[:, :, tq:].view(np.uint16))
    assert np.array_equal(c.v_res[:, :, : c.tr], v[:, :, tq:].view(np.uint16))


def test_flush_schedule(oracle_lib):
    """The residual flushes exactly when a token arrives with R tokens held."""
    B, H, D, G, R = 1, 1, 32, 32, 64
    c = oracle.OracleCache(B, H, 1, D, 2, G, R, 512)
    z = np.zeros((B, H, D), np.float16)
    trs = []
    for i in range(3 * R + 2):
        c.append(z, z)
        trs.append((c.tq, c.tr))
    assert trs[R - 1] == (0, R)
    assert trs[R] == (R, 1)
    assert trs[2 * R] == (2 * R, 1)
    assert c.flushes == 3


def test_capacity_error_leaves_state(oracle_lib):
    B, H, D, G, R = 1, 1, 32, 32, 32
    c = oracle.OracleCache(B, H, 1, D, 2, G, R, 64)
    z = np.zeros((B, H, D), np.float16)
    for _ in range(2 * R + 1):
        c.append(z, z)
    assert (c.tq, c.tr) == (64, 1)
    for _ in range(R - 1):
        c.append(z, z)
    with pytest.raises(oracle.oracle.OracleError, match="ECAPACITY"):
        c.append(z, z)
    assert (c.tq, c.tr) == (64, R)


def test_streaming_workload_prefix(oracle_lib):
    """A few steps of the streaming workload's value model on one batch
    entry: each flush quantizes the tokens in arrival order."""
    w = synth.WORKLOADS["stream_b64_2bit"].with_(batch=1, kv_heads=2, q_heads=2, context=160,
                                                 tq=32)
    k, v = synth.kv(w)
    c = oracle.OracleCache(1, 2, 1, 128, w.bits, w.group, w.residual, 512)
    c.prefill(k, v, w.tq)
    ks, vs = [k], [v]
    for s in range(1, 10):
        kn, vn = synth.new_token(w, s)
        c.append(kn, vn)
        ks.append(kn[:, :, None])
        vs.append(vn[:, :, None])
    assert (c.tq, c.tr) == (160, 9)
    kk = np.concatenate(ks, axis=2)
    ck, _, _ = oracle.quantize_k(kk, w.bits, w.group, 512, ntok=160)
    assert np.array_equal(unpack_k(c.k_codes, 2, 160, 128), unpack_k(ck, 2, 160, 128))

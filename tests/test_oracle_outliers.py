"""Pins of the oracle's key-outlier isolation (dense-and-sparse keys).

Page: "KVQuant: Towards 10 Million Context Length LLM Inference with KV Cache
Quantization" (codewithpapers.app paper page, abstract): outliers are
isolated separately for each vector so that they do not skew the
quantization range.  Reading pinned here: the vector is one key group (one
channel over G tokens); its n_out entries of largest magnitude (ties: lower
position) are kept exactly, the rest are quantized over their own range, and
outlier positions carry code 0.  The pins rest on hand-derived cases, a
brute-force selection by sorting, an identity with the plain quantizer, and
attention on caches that this encoding represents exactly.
"""
import json
import os

import numpy as np
import pytest

import oracle
from tests.helpers import attention_f64, dequant_k_sparse, dequant_v, unpack_k, unpack_outliers

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "outlier_worked_examples.json")
CASES = json.load(open(GOLDEN))["cases"]


def _k_column(values, pad, G, D=128, channel=5):
    col = np.full(G, pad, np.float32)
    col[: len(values)] = values
    k = np.zeros((1, 1, G, D), np.float16)
    k[0, 0, :, channel] = col.astype(np.float16)
    return k


@pytest.mark.parametrize("case", CASES, ids=lambda c: c["name"])
@pytest.mark.parametrize("G", [32, 64])
def test_worked_examples(oracle_lib, case, G):
    bits, n, vals = case["bits"], case["n_out"], case["values"]
    k = _k_column(vals, case["pad"], G)
    codes, s, z, outl = oracle.quantize_k(k, bits, G, cap=64, n_out=n)
    assert s[0, 0, 0, 5] == case["scale"] and z[0, 0, 0, 5] == case["zero"]
    c = unpack_k(codes, bits, G, 128)[0, 0, :, 5]
    assert list(c[: len(vals)]) == case["codes"]
    assert np.all(c[len(vals):] == case["pad_code"])
    assert list(outl[0, 0, 0, :, 5]) == case["words"]
    # an all-zero channel: every magnitude ties, so positions 0 .. n-1 are
    # isolated (value +0) and the dense part is constant 0
    assert list(outl[0, 0, 0, :, 7]) == [j << 16 for j in range(n)]
    assert s[0, 0, 0, 7] == 0 and z[0, 0, 0, 7] == 0


def _brute_positions(x, n):
    """Positions of the n largest |x| (ties: lower position), sorted."""
    order = np.lexsort((np.arange(len(x)), -np.abs(x.astype(np.float64))))
    return sorted(order[:n].tolist())


@pytest.mark.parametrize("n_out", [1, 2, 4, 7])
@pytest.mark.parametrize("G", [32, 64])
def test_selection_brute_force(oracle_lib, n_out, G):
    rng = np.random.default_rng(100 + n_out + G)
    D, T = 64, 2 * G
    # small integers of both signs: magnitudes tie often
    k = rng.integers(-6, 7, (2, 2, T, D)).astype(np.float16)
    k[0, 0, :G, 3] = 0                                # every entry tied
    k[1, 1, G:, 9] = np.float16(-0.0)                 # signed zeros tie with +0
    codes, s, z, outl = oracle.quantize_k(k, 2, G, cap=T, n_out=n_out)
    pos, val = unpack_outliers(outl)
    for b in range(2):
        for h in range(2):
            for g in range(T // G):
                for d in range(D):
                    x = k[b, h, g * G:(g + 1) * G, d]
                    want = _brute_positions(x, n_out)
                    assert pos[b, h, g, :, d].tolist() == want, (b, h, g, d)
                    got = val[b, h, g, :, d].view(np.uint16)
                    assert np.array_equal(got, x[want].view(np.uint16))


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("n_out", [1, 3])
@pytest.mark.parametrize("meta_half", [False, True])
def test_dense_part_is_plain_quantizer(oracle_lib, bits, n_out, meta_half):
    """Quantizing with isolation equals the plain quantizer on the group whose
    outlier entries are replaced by the dense part's minimum (a value that is
    in range and encodes to 0), with code 0 at the outlier positions.
    Including outliers in the range, or coding them, breaks this."""
    G, D, T = 32, 64, 128
    rng = np.random.default_rng(bits * 10 + n_out)
    k = rng.standard_normal((1, 2, T, D)).astype(np.float32)
    spikes = rng.random((1, 2, T, D)) < 0.04
    k = np.where(spikes, k * 30, k).astype(np.float16)
    codes, s, z, outl = oracle.quantize_k(k, bits, G, cap=T, n_out=n_out, meta_half=meta_half)
    pos, _ = unpack_outliers(outl)
    k2 = k.copy()
    mask = np.zeros(k.shape, bool)
    for g in range(T // G):
        for j in range(n_out):
            t = g * G + pos[0, :, g, j, :]                  # [H][D]
            for h in range(2):
                mask[0, h, t[h], np.arange(D)] = True
    for g in range(T // G):
        blk = k[:, :, g * G:(g + 1) * G].astype(np.float32)
        dense_min = np.where(mask[:, :, g * G:(g + 1) * G], np.inf, blk).min(axis=2)
        fill = np.broadcast_to(dense_min[:, :, None, :], blk.shape).astype(np.float16)
        k2[:, :, g * G:(g + 1) * G] = np.where(mask[:, :, g * G:(g + 1) * G], fill,
                                               k[:, :, g * G:(g + 1) * G])
    codes2, s2, z2 = oracle.quantize_k(k2, bits, G, cap=T, meta_half=meta_half)
    assert np.array_equal(s.view(np.uint8), s2.view(np.uint8))
    assert np.array_equal(z.view(np.uint8), z2.view(np.uint8))
    c, c2 = unpack_k(codes, bits, T, D), unpack_k(codes2, bits, T, D)
    assert np.all(c[mask] == 0)
    assert np.array_equal(c[~mask], c2[~mask])


def _lossless_cache(B, H, r, D, G, R, T, tq, n_out, seed):
    """Keys whose every (group, channel) is a constant with at most n_out
    larger-magnitude entries, and values constant over every (token,
    channel group): the dense-and-sparse codes represent them exactly."""
    rng = np.random.default_rng(seed)
    base = (rng.integers(-4, 5, (B, H, T // G, D)) / 4.0).astype(np.float16)   # |c| <= 1
    k = np.repeat(base, G, axis=2).astype(np.float16)
    for b in range(B):
        for h in range(H):
            for g in range(T // G):
                for d in range(D):
                    m = rng.integers(0, n_out + 1)                  # 0 .. n_out spikes
                    idx = rng.choice(G, m, replace=False)
                    k[b, h, g * G + idx, d] = (rng.choice([-1, 1], m) *
                                               rng.uniform(2, 40, m)).astype(np.float16)
    vb = rng.standard_normal((B, H, T, D // G)).astype(np.float16)
    v = np.repeat(vb, G, axis=3)
    q = rng.standard_normal((B, H * r, D)).astype(np.float16)
    return k, v, q


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("n_out", [1, 2])
def test_lossless_attention_closed_form(oracle_lib, bits, n_out):
    """On caches the encoding represents exactly, the oracle's decode equals
    plain binary64 attention over the raw keys and values (a dropped,
    misplaced or sign-flipped outlier changes the result)."""
    B, H, r, D, G, R = 2, 2, 2, 64, 32, 32
    T, tq = 160, 128
    k, v, q = _lossless_cache(B, H, r, D, G, R, T, tq, n_out, seed=bits * 7 + n_out)
    c = oracle.OracleCache(B, H, r, D, bits, G, R, cap=128, n_out=n_out)
    c.prefill(k, v, tq)
    scale = 0.125
    got = c.decode(q, scale)
    want = attention_f64(q, k, v, scale)
    assert np.abs(got - want).max() <= 1e-12 * max(1.0, np.abs(want).max())
    # the spikes matter: keys read as code 0 (the dense zero) at the outlier
    # positions give a clearly different result
    c.k_outl[:] = 0xFFFF0000        # positions no token has: outliers dropped
    assert np.abs(c.decode(q, scale) - want).max() > 1e-3


@pytest.mark.parametrize("bits", [2, 3])
def test_decode_matches_helper_dequant(oracle_lib, bits):
    """Decode on a random cache with isolated outliers equals attention over
    the keys re-read from the documented layouts by the test helpers."""
    B, H, r, D, G, R, T, tq, n_out = 1, 2, 4, 128, 32, 64, 224, 192, 2
    rng = np.random.default_rng(3 + bits)
    k = rng.standard_normal((B, H, T, D)).astype(np.float32)
    k = np.where(rng.random(k.shape) < 0.03, 25 * k, k).astype(np.float16)
    v = rng.standard_normal((B, H, T, D)).astype(np.float16)
    q = rng.standard_normal((B, H * r, D)).astype(np.float16)
    c = oracle.OracleCache(B, H, r, D, bits, G, R, cap=256, n_out=n_out, meta_half=True)
    c.prefill(k, v, tq)
    kd = dequant_k_sparse(c.k_codes, c.ks.view(np.float16), c.kz.view(np.float16), c.k_outl,
                          bits, G, tq, D)
    vd = dequant_v(c.v_codes, c.vs.view(np.float16), c.vz.view(np.float16), bits, G, tq, D)
    kf = np.concatenate([kd, k[:, :, tq:].astype(np.float64)], axis=2)
    vf = np.concatenate([vd, v[:, :, tq:].astype(np.float64)], axis=2)
    scale = float(np.float32(0.088))          # the oracle takes a binary32 scale
    want = attention_f64(q, kf, vf, scale)
    got = c.decode(q, scale)
    assert np.abs(got - want).max() <= 1e-12 * np.abs(want).max()


def test_isolation_shrinks_the_dense_range(oracle_lib):
    """A spike no longer sets the group's scale: every dense entry then
    reconstructs within half a (smaller) step."""
    G, D, T, bits = 32, 64, 64, 2
    rng = np.random.default_rng(11)
    k = rng.standard_normal((1, 1, T, D)).astype(np.float32)
    k[0, 0, 5, :] = 80.0                       # one spike per group-0 column
    k = k.astype(np.float16)
    _, s0, _ = oracle.quantize_k(k, bits, G, cap=T)
    codes, s1, z1, outl = oracle.quantize_k(k, bits, G, cap=T, n_out=1)
    assert np.all(s1[0, 0, 0] < s0[0, 0, 0] / 5)
    kd = dequant_k_sparse(codes, s1, z1, outl, bits, G, T, D)
    err = np.abs(kd - k.astype(np.float64))
    step = np.repeat(s1.astype(np.float64), G, axis=2)
    assert np.all(err <= step / 2 * (1 + 1e-6))
    assert np.all(err[0, 0, 5] == 0)           # the spikes are exact


def test_append_flush_isolates(oracle_lib):
    """Appends that flush the residual isolate outliers of the flushed tokens
    exactly as a direct quantization of those tokens does."""
    B, H, r, D, bits, G, R, n_out = 1, 2, 1, 64, 2, 32, 64, 2
    rng = np.random.default_rng(5)
    T = 64 + 2 * R + 1
    k = (rng.standard_normal((B, H, T, D)) * np.where(rng.random((B, H, T, D)) < 0.05, 20, 1)
         ).astype(np.float16)
    v = rng.standard_normal((B, H, T, D)).astype(np.float16)
    c = oracle.OracleCache(B, H, r, D, bits, G, R, cap=256, n_out=n_out)
    c.prefill(k[:, :, :64], v[:, :, :64], 64)
    for t in range(64, T):
        c.append(k[:, :, t], v[:, :, t])
    assert (c.tq, c.tr, c.flushes) == (64 + R, R, 1) or (c.tq, c.tr) == (64 + 2 * R, 1)
    codes, s, z, outl = oracle.quantize_k(k[:, :, :c.tq], bits, G, cap=256, n_out=n_out)
    assert np.array_equal(c.k_outl, outl)
    assert np.array_equal(c.k_codes, codes)
    assert np.array_equal(c.ks.view(np.uint32), s.view(np.uint32))


def test_outlier_errors(oracle_lib):
    k = np.zeros((1, 1, 32, 64), np.float16)
    with pytest.raises(oracle.oracle.OracleError):
        oracle.quantize_k(k, 2, 32, cap=64, n_out=32)          # no dense entry left
    with pytest.raises(oracle.oracle.OracleError):
        oracle.quantize_k(k, 2, 32, cap=64, n_out=-1, outl=np.zeros(16, np.uint32))

"""Pins of the oracle's codec against facts fixed outside the oracle.

Pages: "KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache"
(mlsanity, Abstract) -- keys per channel, values per token, asymmetric
low-bit codes; study.space summary -- key groups span tokens.  The pages print
no formula: the reading pinned here is z = min, s = (max-min)/(2^b-1),
code = RNE((x-z)/s), each step one binary32 operation.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from kv_cache_bit_kivi_amd import synth
from tests.helpers import unpack_k, unpack_v

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "codec_worked_examples.json")


# ---------------------------------------------------------------------------
# binary16 -> binary32 widening, all 65536 patterns against NumPy
def test_half_to_float_exhaustive(oracle_lib):
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.half_to_float(int(b)) for b in bits], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# ---------------------------------------------------------------------------
def _k_group_input(values, G, D=128, channel=5):
    """One (b, h) plane whose channel `channel` holds `values` (padded with
    values[0]) over G tokens; the other channels are constant 0."""
    col = np.full(G, values[0], np.float32)
    col[: len(values)] = values
    k = np.zeros((1, 1, G, D), np.float16)
    k[0, 0, :, channel] = col.astype(np.float16)
    return k


def _v_group_input(values, G, D=64, token=3, group=1):
    row = np.full(G, values[0], np.float32)
    row[: len(values)] = values
    v = np.zeros((1, 1, 64, D), np.float16)
    v[0, 0, token, group * G:(group + 1) * G] = row.astype(np.float16)
    return v


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
@pytest.mark.parametrize("G", [32, 64])
def test_worked_examples_keys(oracle_lib, case, G):
    bits, vals = case["bits"], case["values"]
    k = _k_group_input(vals, G)
    codes, s, z = oracle.quantize_k(k, bits, G, cap=64 if G <= 64 else G)
    c = unpack_k(codes, bits, G, 128)[0, 0, :, 5]
    assert s[0, 0, 0, 5] == case["scale"] and z[0, 0, 0, 5] == case["zero"]
    assert list(c[: len(vals)]) == case["codes"]
    # padding repeats values[0], whose code is codes[0]
    assert np.all(c[len(vals):] == case["codes"][0])


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_worked_examples_values(oracle_lib, case):
    bits, vals, G = case["bits"], case["values"], 32
    v = _v_group_input(vals, G)
    codes, s, z = oracle.quantize_v(v, bits, G, cap=64)
    c = unpack_v(codes, bits, 64, 64)[0, 0, 3, G:2 * G]
    assert s[0, 0, 3, 1] == case["scale"] and z[0, 0, 3, 1] == case["zero"]
    assert list(c[: len(vals)]) == case["codes"]


# ---------------------------------------------------------------------------
# constant groups dequantize exactly
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_constant_groups_exact(oracle_lib, bits):
    G, D, T = 32, 64, 128
    rng = np.random.default_rng(7)
    # keys: each (group, channel) constant over its G tokens
    kv = rng.standard_normal((1, 2, T // G, D)).astype(np.float16)
    k = np.repeat(kv, G, axis=2)
    codes, s, z = oracle.quantize_k(k, bits, G, cap=T)
    assert np.all(s == 0) and np.all(codes == 0)
    assert np.array_equal(z, kv.astype(np.float32))
    # values: each (token, channel-group) constant over its G channels
    vv = rng.standard_normal((1, 2, T, D // G)).astype(np.float16)
    v = np.repeat(vv, G, axis=3)
    codes, s, z = oracle.quantize_v(v, bits, G, cap=T)
    assert np.all(s == 0) and np.all(codes == 0)
    assert np.array_equal(z, vv.astype(np.float32))


def test_axes_keys_per_channel_values_per_token(oracle_lib):
    """A key tensor constant along tokens (per channel) quantizes exactly only
    if groups run over tokens; a value tensor constant along channels only if
    groups run over channels.  Swapping the axes fails this test."""
    G, D, T = 32, 64, 64
    rng = np.random.default_rng(3)
    k = np.broadcast_to(rng.standard_normal((1, 1, 1, D)).astype(np.float16), (1, 1, T, D)).copy()
    codes, s, z = oracle.quantize_k(k, 2, G, cap=T)
    assert np.all(s == 0)
    codes, s, z = oracle.quantize_v(k, 2, G, cap=T)  # same tensor, per-token groups
    assert np.all(s > 0)
    v = np.broadcast_to(rng.standard_normal((1, 1, T, 1)).astype(np.float16), (1, 1, T, D)).copy()
    codes, s, z = oracle.quantize_v(v, 2, G, cap=T)
    assert np.all(s == 0)
    codes, s, z = oracle.quantize_k(v, 2, G, cap=T)
    assert np.all(s > 0)


def test_outlier_channel_isolated(oracle_lib):
    """Per-channel key groups: scaling one channel by 100 changes that
    channel's scale by 100 and leaves every other channel's scale/codes."""
    w = synth.Workload("t", 1, 2, 2, 64, 128, 2, 32, 32, 128, 0, 11)
    k, _ = synth.kv(w)
    k2 = k.copy()
    k2[..., 17] = (k2[..., 17].astype(np.float32) * 64).astype(np.float16)
    c1, s1, z1 = oracle.quantize_k(k, 2, 32, cap=128)
    c2, s2, z2 = oracle.quantize_k(k2, 2, 32, cap=128)
    other = np.arange(64) != 17
    assert np.array_equal(s1[..., other], s2[..., other])
    u1, u2 = unpack_k(c1, 2, 128, 64), unpack_k(c2, 2, 128, 64)
    assert np.array_equal(u1[..., other], u2[..., other])
    assert np.array_equal(s2[..., 17], s1[..., 17] * 64)   # power of two: exact
    assert np.array_equal(u1[..., 17], u2[..., 17])


# ---------------------------------------------------------------------------
def _groups_keys(x16, G):
    """[B][H][T][D] -> list of per-(b,h,g,d) groups, as float64 [N][G]."""
    B, H, T, D = x16.shape
    return x16.astype(np.float64).reshape(B, H, T // G, G, D).transpose(0, 1, 2, 4, 3).reshape(-1, G)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("G", [32, 64, 128])
def test_error_bound_and_extremes(oracle_lib, bits, G):
    """|x - (c*s + z)| <= s/2 (plus binary32 slack); the group minimum gets
    code 0 and the maximum gets 2^b - 1."""
    D, T = 128, 256
    x = synth.random_fp16(G * bits, (2, 2, T, D), scale=3.0)
    x[0, 0, :, 7] *= np.float16(10)
    codes, s, z = oracle.quantize_k(x, bits, G, cap=T)
    c = unpack_k(codes, bits, T, D)
    qmax = (1 << bits) - 1
    xs = _groups_keys(x, G)
    cs = c.reshape(2, 2, T // G, G, D).transpose(0, 1, 2, 4, 3).reshape(-1, G)
    ss = s.astype(np.float64).reshape(-1)
    zs = z.astype(np.float64).reshape(-1)
    xhat = cs * ss[:, None] + zs[:, None]
    err = np.abs(xs - xhat)
    assert np.all(err <= ss[:, None] * (0.5 + 2.0 ** -18))
    assert np.all(cs >= 0) and np.all(cs <= qmax)
    assert np.all(cs[np.arange(len(xs)), xs.argmin(1)] == 0)
    assert np.all(cs[np.arange(len(xs)), xs.argmax(1)] == qmax)
    assert np.array_equal(zs, xs.min(1))


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_nearest_level_brute_force(oracle_lib, bits):
    """Each code is the nearest of the 2^b levels z + k*s (exact rational
    distances), except within 1e-5 of a tie where binary32 rounding of the
    quotient decides; exact ties go to the even code."""
    G, D, T = 32, 64, 128
    x = synth.random_fp16(100 + bits, (1, 2, T, D))
    codes, s, z = oracle.quantize_k(x, bits, G, cap=T)
    c = unpack_k(codes, bits, T, D)
    qmax = (1 << bits) - 1
    checked = 0
    for h in range(2):
        for g in range(T // G):
            for d in range(0, D, 3):
                sg = Fraction(float(s[0, h, g, d]))
                zg = Fraction(float(z[0, h, g, d]))
                for i in range(G):
                    xv = Fraction(float(x[0, h, g * G + i, d]))
                    vstar = (xv - zg) / sg
                    k = int(vstar)  # floor, vstar >= 0
                    frac = vstar - k
                    if abs(frac - Fraction(1, 2)) < Fraction(1, 100000):
                        continue
                    expect = min(k + (1 if frac > Fraction(1, 2) else 0), qmax)
                    assert c[0, h, g * G + i, d] == expect
                    checked += 1
    assert checked > 2000


def _f32(x: Fraction) -> Fraction:
    """Round an exact rational to the nearest binary32 (ties to even)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    q = Fraction(2) ** (e - 23)           # spacing of binary32 at a
    m = a / q
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * q


def _emulate_group(vals, bits):
    xs = [Fraction(float(v)) for v in vals]
    mn, mx = min(xs), max(xs)
    if mn == mx:
        return 0.0, float(mn), [0] * len(xs)
    s = _f32(_f32(mx - mn) / ((1 << bits) - 1))
    codes = []
    for xv in xs:
        v = _f32(_f32(xv - mn) / s)
        n = v.numerator // v.denominator
        rem = v - n
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
            n += 1
        codes.append(min(n, (1 << bits) - 1))
    return float(s), float(mn), codes


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_exact_rational_emulation(oracle_lib, bits):
    """Bit-exact agreement with an exact-rational emulation of each binary32
    step (subtract, divide, round half to even)."""
    G, D, T = 32, 32, 64
    x = synth.random_fp16(300 + bits, (1, 1, T, D), scale=0.7)
    x[0, 0, :, 3] *= np.float16(40)
    codes, s, z = oracle.quantize_k(x, bits, G, cap=T)
    c = unpack_k(codes, bits, T, D)
    for g in range(T // G):
        for d in range(D):
            es, ez, ec = _emulate_group(x[0, 0, g * G:(g + 1) * G, d], bits)
            assert np.float32(es) == s[0, 0, g, d]
            assert np.float32(ez) == z[0, 0, g, d]
            assert list(c[0, 0, g * G:(g + 1) * G, d]) == ec
    codes, s, z = oracle.quantize_v(x, bits, G, cap=T)
    c = unpack_v(codes, bits, T, D)
    for t in range(T):
        es, ez, ec = _emulate_group(x[0, 0, t, :G], bits)
        assert np.float32(es) == s[0, 0, t, 0] and np.float32(ez) == z[0, 0, t, 0]
        assert list(c[0, 0, t, :G]) == ec


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("k", [-3, 1, 4])
def test_power_of_two_scaling(oracle_lib, bits, k):
    """x -> 2^k x keeps every code and scales s, z by exactly 2^k."""
    G, D, T = 32, 64, 128
    x = synth.random_fp16(500 + bits, (1, 2, T, D))
    x = np.where(np.abs(x.astype(np.float32)) < 2.0 ** -10, np.float16(0.5), x)  # stay normal
    y = (x.astype(np.float32) * np.float32(2.0 ** k)).astype(np.float16)
    assert np.array_equal(y.astype(np.float32), x.astype(np.float32) * 2.0 ** k)
    for fn, unpack in ((oracle.quantize_k, unpack_k), (oracle.quantize_v, unpack_v)):
        c1, s1, z1 = fn(x, bits, G, cap=T)
        c2, s2, z2 = fn(y, bits, G, cap=T)
        assert np.array_equal(unpack(c1, bits, T, D), unpack(c2, bits, T, D))
        assert np.array_equal(s2, s1 * np.float32(2.0 ** k))
        assert np.array_equal(z2, z1 * np.float32(2.0 ** k))


def _bit_slots(bits, n, p):
    """[(word, bit, value bit)] that position p of a row of n codes occupies,
    written out from the documented layout (independent of helpers.py)."""
    beta = 4 * ((p % 32 % 16) // 2) + 2 * ((p % 32) // 16) + p % 2
    if bits == 1:
        return [(p // 32, beta, 0)]
    if bits == 3:
        return [(p // 16, 2 * (p % 16), 0), (p // 16, 2 * (p % 16) + 1, 1),
                (n // 16 + p // 32, beta, 2)]
    E = 32 // bits
    return [(p // E, bits * (p % E) + i, i) for i in range(bits)]


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_packed_bit_positions(oracle_lib, bits):
    """Codes land at the documented bit positions.  Inputs are exactly the
    integer levels (scale 1, zero 0), so the code of (t, d) is known in
    advance without running the quantizer's arithmetic."""
    G, D, T = 32, 64, 128
    qmax = (1 << bits) - 1
    t = np.arange(T)[:, None]
    d = np.arange(D)[None, :]
    base = (3 * t + 5 * d) % (qmax + 1)
    lk = base.copy()
    lk[::G, :] = 0             # every key group (tokens of a channel) spans 0..qmax
    lk[1::G, :] = qmax
    ck, sk, zk = oracle.quantize_k(lk.astype(np.float16)[None, None], bits, G, cap=T)
    assert np.all(sk == 1) and np.all(zk == 0)
    for tt in (0, 5, 77, 127):
        for dd in (0, 1, 15, 16, 31, 32, D - 1):
            got = sum(((int(ck[0, 0, tt, w]) >> bit) & 1) << vb
                      for w, bit, vb in _bit_slots(bits, D, dd))
            assert got == lk[tt, dd], (tt, dd)
    lv = base.copy()
    lv[:, ::G] = 0             # every value group (channels of a token) spans 0..qmax
    lv[:, 1::G] = qmax
    cv, sv, zv = oracle.quantize_v(lv.astype(np.float16)[None, None], bits, G, cap=T)
    assert np.all(sv == 1) and np.all(zv == 0)
    for tt in (0, 5, 15, 16, 31, 32, 63, 64, 100, 127):
        for dd in (0, 7, D - 1):
            got = sum(((int(cv[0, 0, tt // 64, dd, w]) >> bit) & 1) << vb
                      for w, bit, vb in _bit_slots(bits, 64, tt % 64))
            assert got == lv[tt, dd], (tt, dd)
    # every word bit is used exactly once per row (the layout is a bijection)
    for n in (D, 64):
        seen = set()
        for pp in range(n):
            for w, bit, _ in _bit_slots(bits, n, pp):
                assert (w, bit) not in seen
                seen.add((w, bit))
        assert len(seen) == n * bits


def test_offset_and_stride(oracle_lib):
    """Quantizing tokens [0, n) of a strided input into offset o equals
    quantizing the same tokens into offset 0, moved by o tokens."""
    G, D = 32, 64
    x = synth.random_fp16(9, (2, 3, 160, D))
    for fn, unpack in ((oracle.quantize_k, unpack_k), (oracle.quantize_v, unpack_v)):
        c0, s0, z0 = fn(x, 2, G, cap=256, ntok=96, dst_off=0)
        c1, s1, z1 = fn(x, 2, G, cap=256, ntok=96, dst_off=96)
        u0, u1 = unpack(c0, 2, 256, D), unpack(c1, 2, 256, D)
        assert np.array_equal(u0[:, :, :96], u1[:, :, 96:192])
        if fn is oracle.quantize_k:
            assert np.array_equal(s0[:, :, :3], s1[:, :, 3:6])
        else:
            assert np.array_equal(s0[:, :, :96], s1[:, :, 96:192])


def test_error_codes(oracle_lib):
    x = synth.random_fp16(1, (1, 1, 64, 64))
    with pytest.raises(oracle.oracle.OracleError, match="EINVAL"):
        oracle.quantize_k(x, 5, 32, cap=64)
    with pytest.raises(oracle.oracle.OracleError, match="EINVAL"):
        oracle.quantize_k(x, 0, 32, cap=64)
    with pytest.raises(oracle.oracle.OracleError, match="ESHAPE"):
        oracle.quantize_k(x, 2, 32, cap=64, ntok=48)
    with pytest.raises(oracle.oracle.OracleError, match="ECAPACITY"):
        oracle.quantize_k(x, 2, 32, cap=64, ntok=64, dst_off=32)


@pytest.mark.parametrize("meta_half", [False, True])
@pytest.mark.parametrize("n_out", [0, 1, 2])
@pytest.mark.parametrize("bits", [1, 2, 4])
def test_key_zeros_are_binary16_values(oracle_lib, bits, n_out, meta_half):
    """A key zero is the minimum of binary16 inputs (the group's, or of the
    entries left after its outliers), so it is a binary16 value exactly: the
    matrix-core decode takes the zeros as binary16 operands for several heads
    per KV head.  Spiky inputs, a constant group and a group of signed zeros
    included; with outliers the zero is the minimum of the dense rest."""
    G, T, D = 32, 128, 128
    x = synth.spiky_fp16(40 + bits, (1, 2, T, D), rate=0.03, scale=2.0)
    x[0, 0, 0:G, 3] = np.float16(0.7)                       # constant group
    x[0, 0, G:2 * G, 5] = np.float16(-0.0)
    x[0, 0, G + 7, 5] = np.float16(0.0)                     # signed zeros
    out = oracle.quantize_k(x, bits, G, cap=T, meta_half=meta_half, n_out=n_out)
    z = out[2]
    zf = (z.view(np.float16).astype(np.float64) if meta_half else z.astype(np.float64)).reshape(-1)
    assert np.array_equal(zf, zf.astype(np.float16).astype(np.float64))
    xs = _groups_keys(x, G)                                  # [groups][G], same order
    if n_out == 0:
        assert np.array_equal(zf, xs.min(1))
    else:
        # the n_out entries of largest magnitude (lower token first) leave the range
        order = np.argsort(-np.abs(xs), axis=1, kind="stable")[:, :n_out]
        mask = np.ones_like(xs, dtype=bool)
        np.put_along_axis(mask, order, False, axis=1)
        dense_min = np.where(mask, xs, np.inf).min(1)
        assert np.array_equal(zf, dense_min)

"""Pins of the oracle's pre-RoPE key path.

Page: "KVQuant: Towards 10 Million Context Length LLM Inference with KV Cache
Quantization" (codewithpapers.app, abstract): keys are quantized before the
rotary positional embedding.  Reading pinned here: the cache holds pre-RoPE
keys; decode rotates each dequantized key at its token index with the
rotate-half embedding (pairs (i, i + D/2), frequency theta^(-2i/D)); queries
arrive already rotated.  The pins: the Llama rotary embedding of the
`transformers` library applied to the keys, the same rotation written as
complex multiplication, and special cases."""
import numpy as np
import pytest
import torch

import oracle
from tests.helpers import attention_f64, dequant_k, dequant_v


def hf_rope_keys(k, theta):
    """Keys k [B][H][T][D] rotated at positions 0..T-1 by the Llama rotary
    embedding of `transformers` (rotate-half form)."""
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb
    B, H, T, D = k.shape
    cfg = LlamaConfig(hidden_size=D * 2, num_attention_heads=2, rope_theta=float(theta))
    emb = LlamaRotaryEmbedding(config=cfg)
    kt = torch.from_numpy(np.ascontiguousarray(k, np.float64))
    cos, sin = emb(kt, torch.arange(T)[None])
    _, kr = apply_rotary_pos_emb(kt, kt, cos, sin, unsqueeze_dim=1)
    return kr.numpy()


def complex_rope_keys(k, theta):
    """The same rotation as complex multiplication: (k_i + j k_{i+D/2}) *
    exp(j * t * theta^(-2i/D))."""
    D = k.shape[-1]
    h = D // 2
    T = k.shape[2]
    f = np.power(float(theta), -2.0 * np.arange(h) / D)
    e = np.exp(1j * np.outer(np.arange(T), f))            # [T][h]
    z = (k[..., :h].astype(np.float64) + 1j * k[..., h:].astype(np.float64)) * e
    return np.concatenate([z.real, z.imag], axis=-1)


def _cache(B, H, r, D, bits, G, R, T, tq, theta, seed, mh=False):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, H, T, D)).astype(np.float16)
    v = rng.standard_normal((B, H, T, D)).astype(np.float16)
    q = rng.standard_normal((B, H * r, D)).astype(np.float16)
    cap = max(64, (tq + 63) // 64 * 64)
    c = oracle.OracleCache(B, H, r, D, bits, G, R, cap, meta_half=mh, rope_theta=theta)
    c.prefill(k, v, tq)
    return c, k, v, q


@pytest.mark.parametrize("theta", [10000.0, 500000.0, 2.0])
@pytest.mark.parametrize("D", [64, 128])
def test_residual_keys_match_library_rope(oracle_lib, theta, D):
    """A residual-only cache (exact fp16 keys): decode equals attention over
    the keys rotated by the library's Llama rotary embedding."""
    B, H, r, G, R, T = 1, 2, 2, 32, 128, 120
    c, k, v, q = _cache(B, H, r, D, 2, G, R, T, 0, theta, seed=int(D + theta) % 1000)
    scale = float(np.float32(0.125))
    want = attention_f64(q, hf_rope_keys(k, theta), v, scale)
    got = c.decode(q, scale)
    # the library computes its angles in binary32: allow ~1e-5 of angle error
    assert np.abs(got - want).max() <= 2e-4 * np.abs(want).max()


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("meta_half", [False, True])
def test_quantized_keys_match_complex_rope(oracle_lib, bits, meta_half):
    """Quantized + residual keys: decode equals attention over the keys
    re-read from the documented layout by the test helpers, rotated as
    complex numbers (binary64)."""
    B, H, r, D, G, R, T, tq = 2, 2, 1, 64, 32, 64, 200, 160
    c, k, v, q = _cache(B, H, r, D, bits, G, R, T, tq, 10000.0, seed=bits, mh=meta_half)
    mt = np.float16 if meta_half else np.float32
    kd = dequant_k(c.k_codes, c.ks.view(mt), c.kz.view(mt), bits, G, tq, D)
    vd = dequant_v(c.v_codes, c.vs.view(mt), c.vz.view(mt), bits, G, tq, D)
    kf = np.concatenate([kd, k[:, :, tq:].astype(np.float64)], axis=2)
    vf = np.concatenate([vd, v[:, :, tq:].astype(np.float64)], axis=2)
    scale = float(np.float32(0.125))
    want = attention_f64(q, complex_rope_keys(kf, 10000.0), vf, scale)
    got = c.decode(q, scale)
    assert np.abs(got - want).max() <= 1e-12 * np.abs(want).max()


def test_library_and_complex_forms_agree():
    """The two independent formulations of the rotation agree (so the pins
    above pin the same embedding)."""
    rng = np.random.default_rng(0)
    k = rng.standard_normal((1, 1, 300, 128))
    a, b = hf_rope_keys(k, 10000.0), complex_rope_keys(k, 10000.0)
    assert np.abs(a - b).max() < 1e-4


def test_theta_zero_is_plain_and_positions_matter(oracle_lib):
    """rope_theta = 0 is the plain path; with rope the result differs, and a
    cache whose keys are rotated by the test before caching, decoded without
    rope, differs from the pre-RoPE cache only by the key quantization."""
    B, H, r, D, G, R, T, tq = 1, 2, 1, 64, 32, 64, 160, 128
    c, k, v, q = _cache(B, H, r, D, 2, G, R, T, tq, 0.0, seed=3)
    c2, _, _, _ = _cache(B, H, r, D, 2, G, R, T, tq, 10000.0, seed=3)
    plain = oracle.OracleCache(B, H, r, D, 2, G, R, 128)
    plain.prefill(k, v, tq)
    assert np.array_equal(c.decode(q, 0.125), plain.decode(q, 0.125))
    assert np.abs(c2.decode(q, 0.125) - plain.decode(q, 0.125)).max() > 1e-3


def test_rope_first_position_identity(oracle_lib):
    """Token 0 is not rotated: with a single cached token the attention is
    its value either way, and with two tokens whose second key is zero the
    first token's score is the plain one."""
    B, H, r, D, G, R = 1, 1, 1, 64, 32, 32
    rng = np.random.default_rng(9)
    k = rng.standard_normal((B, H, 2, D)).astype(np.float16)
    k[:, :, 1] = 0
    v = rng.standard_normal((B, H, 2, D)).astype(np.float16)
    q = rng.standard_normal((B, H * r, D)).astype(np.float16)
    a = oracle.OracleCache(B, H, r, D, 2, G, R, 64, rope_theta=10000.0)
    b = oracle.OracleCache(B, H, r, D, 2, G, R, 64)
    a.prefill(k, v, 0)
    b.prefill(k, v, 0)
    assert np.allclose(a.decode(q, 0.2), b.decode(q, 0.2), rtol=0, atol=1e-15)


def test_rope_errors(oracle_lib):
    B, H, r, D, G, R = 1, 1, 1, 64, 32, 32
    k = np.zeros((B, H, 4, D), np.float16)
    for bad in (-1.0, float("inf"), float("nan")):
        c = oracle.OracleCache(B, H, r, D, 2, G, R, 64, rope_theta=bad)
        c.prefill(k, k, 0)
        with pytest.raises(oracle.oracle.OracleError):
            c.decode(np.zeros((B, H * r, D), np.float16), 0.1)

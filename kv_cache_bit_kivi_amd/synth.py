"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers and describes workload shapes; it holds
none of the method's arithmetic and imports nothing from the library or the
oracle.  Both sides of every parity check receive the same arrays from here.

Value model.  The KIVI summary page reports that the key cache has a few
channels of large magnitude while the value cache shows no outlier pattern
("KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache", study.space
summary).  Trained-model activations are not available, so:
  K = N(0, 1) with ``n_outliers`` fixed channels per KV head multiplied by 10,
  V = N(0, 1), q = N(0, 1), each drawn in binary32 and rounded to binary16
  (round to nearest even).
Sporadic key outliers (``key_spikes`` > 0, for the per-vector outlier
isolation of "KVQuant: Towards 10 Million Context Length LLM Inference with KV
Cache Quantization", codewithpapers.app page, abstract): each key entry is
independently multiplied by 20 with probability ``key_spikes`` (a seeded mask
stream of its own), so that single entries, not whole channels, stand out.
Every (batch, head) plane has its own PCG64 stream keyed by
SeedSequence([seed, stream, b, h]) so any single head can be regenerated alone.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# stream ids of SeedSequence([seed, stream, ...])
S_OUTLIER, S_K, S_V, S_Q, S_KNEW, S_VNEW, S_QNEW, S_LEN, S_SPIKE, S_SPIKENEW = range(10)
SPIKE_FACTOR = 20.0


@dataclass(frozen=True)
class Workload:
    """Shape of one decode workload (a single attention layer)."""
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    context: int        # tokens in the cache at the decode call
    bits: int
    group: int
    residual: int
    tq: int             # quantized tokens at the decode call (multiple of group)
    n_outliers: int
    seed: int
    steps: int = 0      # streaming decode steps after the prefill
    min_context: int = 0   # > 0: ragged batch, contexts drawn in [min_context, context]
    key_spikes: float = 0.0   # probability of a sporadic x20 key entry

    @property
    def gqa(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def tr(self) -> int:
        return self.context - self.tq

    @property
    def ragged(self) -> bool:
        return self.min_context > 0

    def contexts(self) -> np.ndarray:
        """Per-sequence context lengths: all ``context``, or (ragged) drawn
        uniformly from [min_context, context] by a seeded stream."""
        if not self.ragged:
            return np.full(self.batch, self.context, np.int64)
        g = _rng(self.seed, S_LEN)
        return g.integers(self.min_context, self.context + 1, self.batch)

    def tqs(self) -> np.ndarray:
        """Per-sequence quantized lengths (the residual holds the rest)."""
        if not self.ragged:
            return np.full(self.batch, self.tq, np.int64)
        return np.array([_resid_split(int(L), self.residual) for L in self.contexts()])

    @property
    def softmax_scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    def capacity(self, extra_tokens: int = 0) -> int:
        """Quantized-store capacity (tokens) that holds every flush of
        ``extra_tokens`` appended tokens, rounded up to the 64-token tile."""
        need = self.context + extra_tokens + self.residual
        step = max(64, self.group)
        return (need + step - 1) // step * step

    def with_(self, **kw) -> "Workload":
        d = self.__dict__.copy()
        d.update(kw)
        return Workload(**d)


def _resid_split(context: int, residual: int) -> int:
    """tq such that the residual holds ((context-1) mod R)+1 tokens."""
    return context - ((context - 1) % residual + 1)


WORKLOADS = {
    # single head, 512 tokens, every token quantized
    "single_head_512": Workload("single_head_512", 1, 1, 1, 128, 512, 2, 32, 32, 512, 4, 1001),
    # Llama-2-7B-shaped layer: batch 8, 32 MHA heads, context 4096
    "llama2_7b_b8_ctx4096": Workload("llama2_7b_b8_ctx4096", 8, 32, 32, 128, 4096, 2, 32, 128,
                                     _resid_split(4096, 128), 8, 1002),
    # Mistral-7B-shaped layer: batch 32, 32 query / 8 KV heads, context 8192
    "mistral_7b_b32_ctx8192": Workload("mistral_7b_b32_ctx8192", 32, 32, 8, 128, 8192, 2, 32,
                                       128, _resid_split(8192, 128), 8, 1003),
    # streaming: batch 64, 32 heads, prefill 4096 then 256 appended tokens
    "stream_b64_4bit": Workload("stream_b64_4bit", 64, 32, 32, 128, 4096, 4, 32, 128,
                                _resid_split(4096, 128), 8, 1004, steps=256),
    "stream_b64_2bit": Workload("stream_b64_2bit", 64, 32, 32, 128, 4096, 2, 32, 128,
                                _resid_split(4096, 128), 8, 1004, steps=256),
    # long context: batch 1, 32 heads, 262144 tokens
    "long_ctx_262144": Workload("long_ctx_262144", 1, 32, 32, 128, 262144, 2, 32, 128,
                                _resid_split(262144, 128), 8, 1005),
    # ragged serving batch: 16 Llama-2-7B-shaped sequences, contexts uniform in
    # [512, 8192] (each residual at its own fill level)
    "ragged_b16_ctx512_8192": Workload("ragged_b16_ctx512_8192", 16, 32, 32, 128, 8192, 2, 32,
                                       128, _resid_split(8192, 128), 8, 1006, min_context=512),
}


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *key])))


def outlier_channels(w: Workload, h: int) -> np.ndarray:
    return np.sort(_rng(w.seed, S_OUTLIER, h).choice(w.head_dim, w.n_outliers, replace=False))


def _spikes(w: Workload, x: np.ndarray, *key: int) -> None:
    """Multiply a seeded Bernoulli(key_spikes) subset of x's entries by 20."""
    if w.key_spikes > 0:
        m = _rng(w.seed, *key).random(x.shape) < w.key_spikes
        x[m] *= np.float32(SPIKE_FACTOR)


def _plane(w: Workload, stream: int, b: int, h: int, T: int, outliers: bool) -> np.ndarray:
    x = _rng(w.seed, stream, b, h).standard_normal((T, w.head_dim), dtype=np.float32)
    if outliers and w.n_outliers:
        x[:, outlier_channels(w, h)] *= np.float32(10.0)
    if outliers:
        _spikes(w, x, S_SPIKE, b, h)
    return x.astype(np.float16)


def k_plane(w: Workload, b: int, h: int, T: int | None = None) -> np.ndarray:
    """Keys of one (batch, kv-head) plane, [T][D] binary16."""
    return _plane(w, S_K, b, h, w.context if T is None else T, True)


def v_plane(w: Workload, b: int, h: int, T: int | None = None) -> np.ndarray:
    return _plane(w, S_V, b, h, w.context if T is None else T, False)


def kv(w: Workload, T: int | None = None, batches=None):
    """Full K, V arrays [B'][Hkv][T][D] binary16 (B' = len(batches))."""
    T = w.context if T is None else T
    bs = range(w.batch) if batches is None else batches
    k = np.stack([np.stack([k_plane(w, b, h, T) for h in range(w.kv_heads)]) for b in bs])
    v = np.stack([np.stack([v_plane(w, b, h, T) for h in range(w.kv_heads)]) for b in bs])
    return k, v


def query(w: Workload, step: int = 0, batches=None) -> np.ndarray:
    """Decode queries [B'][Hq][D] binary16; step > 0 gives streaming queries."""
    bs = range(w.batch) if batches is None else batches
    out = []
    for b in bs:
        g = _rng(w.seed, S_Q if step == 0 else S_QNEW, step, b)
        out.append(g.standard_normal((w.q_heads, w.head_dim), dtype=np.float32))
    return np.stack(out).astype(np.float16)


def new_token(w: Workload, step: int, batches=None):
    """K and V of the token appended at streaming step ``step`` (>= 1),
    [B'][Hkv][D] binary16, same value model as the prefill."""
    bs = range(w.batch) if batches is None else batches
    ks, vs = [], []
    for b in bs:
        gk = _rng(w.seed, S_KNEW, step, b)
        k = gk.standard_normal((w.kv_heads, w.head_dim), dtype=np.float32)
        for h in range(w.kv_heads):
            if w.n_outliers:
                k[h, outlier_channels(w, h)] *= np.float32(10.0)
        _spikes(w, k, S_SPIKENEW, step, b)
        gv = _rng(w.seed, S_VNEW, step, b)
        ks.append(k)
        vs.append(gv.standard_normal((w.kv_heads, w.head_dim), dtype=np.float32))
    return np.stack(ks).astype(np.float16), np.stack(vs).astype(np.float16)


def random_fp16(seed: int, shape, scale: float = 1.0) -> np.ndarray:
    """Generic seeded N(0, scale^2) binary16 tensor for small test cases."""
    return (_rng(seed, 99).standard_normal(shape, dtype=np.float32) * np.float32(scale)).astype(np.float16)


def spiky_fp16(seed: int, shape, rate: float = 0.02, scale: float = 1.0) -> np.ndarray:
    """random_fp16 with a seeded Bernoulli(rate) subset of entries multiplied
    by 20 (sporadic single-entry outliers)."""
    x = _rng(seed, 99).standard_normal(shape, dtype=np.float32) * np.float32(scale)
    x[_rng(seed, 98).random(shape) < rate] *= np.float32(SPIKE_FACTOR)
    return x.astype(np.float16)

"""KIVI-style asymmetric low-bit KV cache for AMD Instinct MI355X (gfx950).

Per-channel key / per-token value quantization, a full-precision residual of
recent tokens flushed into the quantized store, and decode attention that
reads the packed cache directly -- all in hand-written HIP kernels behind the
C ABI of include/kivi.h.  ``_lib`` binds that ABI; ``cache.KiviCache`` owns
the device buffers (PyTorch tensors) of one layer.
"""
from ._lib import KiviError, lib  # noqa: F401

"""CPU oracle for the KIVI quantized KV cache hot path.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the product package never does.
The arithmetic lives in ``kivi_oracle.c`` (plain single-threaded C); this
module only builds it with gcc, loads it with ctypes and marshals NumPy arrays.
"""
from .oracle import (  # noqa: F401
    OracleCache,
    build,
    decode_attn,
    float_to_half,
    half_to_float,
    load,
    meta_dtype,
    outlier_shape,
    quantize_k,
    quantize_v,
    quantize_v_token,
)

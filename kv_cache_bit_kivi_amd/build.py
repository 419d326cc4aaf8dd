"""Build libkivi.so (all HIP kernels + the C ABI) for gfx950 with hipcc.

Usage: python -m kv_cache_bit_kivi_amd.build   (or build() from Python).
Objects go to <repo>/_build/, the library to kv_cache_bit_kivi_amd/libkivi.so.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkivi.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-I" + INCLUDE, "-I" + CSRC,
    # no packed-fp32 VALU ops anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# per-source extra flags: the codec is a bit-exact contract (no contraction;
# division stays the correctly rounded default); the matrix-core decode
# kernels with stored keys are scheduled for instruction-level parallelism
# (their tile loop is a latency-bound chain; against the default scheduler,
# same box: batch-8 Llama layer 26.39 -> 26.26 us, Mistral-shaped 57.5-58.0 ->
# 57.1-57.3 us, ragged batch 51.3 -> 51.0 us, one and two key outliers per
# group 31.0 -> 30.6 us and 37.9-38.3 -> 37.5-37.7 us, paged store 27.44-27.51
# -> 27.40-27.43 us); the pre-RoPE units keep the default (no gain measured)
_ILP = ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]
EXTRA = {
    "quantize.hip": ["-ffp-contract=off"],
    **{f: _ILP for f in ("decode_mfma.hip", "decode_mfma_ragged.hip", "decode_mfma_paged.hip",
                         "decode_mfma_o1.hip", "decode_mfma_o2.hip", "decode_mfma_ragged_o.hip",
                         "decode_mfma_paged_o.hip")},
}
# (longest compiles first: the pool starts them first)
SOURCES = ["decode_mfma_ragged_o.hip", "decode_mfma_paged_o.hip", "decode_mfma_rope.hip",
           "decode_mfma_ragged_rope.hip", "decode_mfma_paged_rope.hip", "decode_mfma.hip",
           "decode_mfma_ragged.hip", "decode_mfma_paged.hip", "decode_mfma_o1.hip",
           "decode_mfma_o2.hip", "kivi_api.hip", "quantize.hip", "decode_generic.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

"""Decode attention captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

A serving loop can capture the decode launch once and replay it: the kernels
take their lengths as launch arguments, allocate nothing and issue no memset
or host synchronisation, and the shared-tile counter lives in LDS and is set
by each block.  Every replay, with the program's own eager work and
synchronisations between replays, must meet the oracle's bar; a deterministic
cache's replays must equal its eager output bit for bit.  Covered: one split
(direct fp16 output) and several (workspace partials + combine launch), one
and four heads per KV head."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_bit_kivi_amd import synth
from kv_cache_bit_kivi_amd.cache import KiviCache
from tests.gpu_util import ATTN_TOL, announce, dev, host, require_gpu, row_rel_err

pytestmark = pytest.mark.gpu

SCALE = 0.0883883461356163


@pytest.mark.parametrize("r,splits", [(1, 1), (1, 6), (4, 1), (4, 3)])
@pytest.mark.parametrize("deterministic", [False, True])
def test_decode_graph_replays(r, splits, deterministic):
    require_gpu()
    announce(f"decode graph r={r} splits={splits} deterministic={deterministic}")
    B, H, D, bits, G, R = 2, 4, 128, 2, 32, 128
    tq, tr = 1984, 70
    cap = 2176
    seed = 700 + 10 * r + splits
    k = synth.random_fp16(seed, (B, H, tq + tr, D), scale=2.0)
    v = synth.random_fp16(seed + 1, (B, H, tq + tr, D))
    q = synth.random_fp16(seed + 2, (B, H * r, D))
    gc = KiviCache(B, H, r, D, bits, G, R, cap, deterministic=deterministic)
    gc.prefill(dev(k), dev(v), tq)
    oc = oracle.OracleCache(B, H, r, D, bits, G, R, cap)
    oc.prefill(k, v, tq)
    ref = oc.decode(q, SCALE)

    qd = dev(q)
    out = torch.empty_like(qd)
    gc.workspace_for(splits)                 # allocated before the capture
    eager = host(gc.decode(qd, SCALE, out=out, num_splits=splits)).copy()
    assert row_rel_err(eager.astype(np.float64), ref) <= ATTN_TOL

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):            # warm the capture stream once
        gc.decode(qd, SCALE, out=out, num_splits=splits)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gc.decode(qd, SCALE, out=out, num_splits=splits)
    torch.cuda.synchronize()

    scratch = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    for i in range(4):
        out.fill_(float("nan"))              # eager work between replays
        scratch.normal_()
        graph.replay()
        torch.cuda.synchronize()
        got = host(out)
        assert row_rel_err(got.astype(np.float64), ref) <= ATTN_TOL, i
        if deterministic:
            assert np.array_equal(got.view(np.uint16), eager.view(np.uint16)), i

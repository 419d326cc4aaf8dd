#!/usr/bin/env python3
"""Benchmark of the quantized-KV decode hot path on one MI355X.

A step is one decode step of one attention layer of the Llama-2-7B-shaped
workload (batch 8, 32 heads, head_dim 128, 2-bit codes, G = 32, R = 128,
context 4096 at the start of the timed region): append the new token's K/V
(quantizing the full residual into the grouped part when it is full), then
decode attention for every query head, as one kivi_append_decode_attn call
(the append is folded into the decode launch; `--separate` times
kivi_append + kivi_decode_attn instead).  Steps rotate over `--layers`
independent layer caches, by default the model's 32 layers (4.6 GB in total;
fewer for larger layers, within 16 GB), as a decode step of the whole model
visits them, so that no step finds its cache resident in the 256 MB Infinity
Cache left by the previous step.  By default 128 steps per layer are timed
(4096); each layer starts with a full residual, so every layer flushes once
per 128 appends, the method's own rate.

Prints one JSON line: whole-step algorithmic HBM GB/s (value), query-heads/s,
the roofline of the dominant kernel (decode attention with the folded append,
timed with HIP events on the launch stream around windows of `--window`
consecutive calls inside the timed region, windows holding a flush left out)
and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "quantized-KV decode attention: achieved HBM GB/s (% of peak), query-heads/s"


def decode_bytes(B, H, r, D, bits, G, tq, tr, mb=4, n_out=0):
    """Algorithmic bytes of one decode call: packed K/V codes, scale and zero
    of both (mb bytes each: 4 for binary32, 2 for binary16), the key-outlier
    words (n_out 4-byte words per key group and channel), fp16 residual K/V,
    fp16 q and out."""
    per = (2 * tq * D * bits // 8 + (tq // G) * D * 2 * mb + tq * (D // G) * 2 * mb
           + (tq // G) * n_out * D * 4 + 4 * tr * D + 4 * r * D)
    return B * H * per


def append_bytes(B, H, D, bits, G, R, flush, mb=4, n_out=0):
    """Algorithmic bytes of one append: read the new K/V token, write it to
    the residual; a flush reads R residual tokens of K and V and writes their
    codes, scales, zeros and key-outlier words."""
    b = B * H * D * 2 * 2 * 2
    if flush:
        b += B * H * (2 * R * D * 2 + 2 * R * D * bits // 8 + (R // G) * D * 2 * mb
                      + R * (D // G) * 2 * mb + (R // G) * n_out * D * 4)
    return b


# the sources that define the decode kernel and its launch configuration
DECODE_SOURCES = ("decode_mfma_impl.h", "decode_mfma.hip", "decode_mfma_ragged.hip",
                  "decode_mfma_paged.hip", "decode_mfma_o1.hip", "decode_mfma_o2.hip",
                  "decode_mfma_ragged_o.hip", "decode_mfma_paged_o.hip", "decode_mfma_rope.hip",
                  "decode_mfma_ragged_rope.hip", "decode_mfma_paged_rope.hip", "kivi_internal.h",
                  "kivi_api.hip")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        h.update(name.encode())
        h.update(open(os.path.join(ROOT, "kv_cache_bit_kivi_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


DECODE_KERNEL = "decode_mfma_kernel"
# PMC calibration kernel: torch's elementwise bitwise_not over N bytes, a plain
# copy-shaped kernel (reads N bytes, writes N bytes) with a recognisable name
COPY_KERNEL_HINT = "bitwise_not"


def measured_traffic(workload: str):
    """HBM bytes per decode launch from the committed rocprofv3 PMC summary,
    only if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def pmc_summary(fetch_csv: str, write_csv: str, copy_bytes: int, workload: str, command: str):
    """Calibrated HBM traffic of the decode kernel from two rocprofv3 --pmc
    runs (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).  Each counter is
    scaled by bytes / counter of the plain copy kernel that the same run
    timed first (--copy-calibration: reads and writes `copy_bytes`)."""
    import csv

    def per_kernel(path, counter):
        dec, cpy = [], []
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] != counter:
                continue
            v = float(row["Counter_Value"])
            name = row["Kernel_Name"]
            if DECODE_KERNEL in name:
                dec.append(v)
            elif COPY_KERNEL_HINT in name:
                cpy.append(v)
        if not dec or not cpy:
            raise SystemExit(f"{path}: no {counter} rows for the decode or copy kernel")
        return sum(dec) / len(dec), sum(cpy) / len(cpy), len(dec), len(cpy)

    f_dec, f_cpy, nf, ncf = per_kernel(fetch_csv, "FETCH_SIZE")
    w_dec, w_cpy, nw, ncw = per_kernel(write_csv, "WRITE_SIZE")
    k_fetch = copy_bytes / (f_cpy * 1024.0)
    k_write = copy_bytes / (w_cpy * 1024.0)
    read_b = f_dec * 1024.0 * k_fetch
    write_b = w_dec * 1024.0 * k_write
    out = {
        "kernel": DECODE_KERNEL,
        "workload": workload,
        "command": command,
        "fetch_size_kib_per_dispatch": round(f_dec, 1),
        "write_size_kib_per_dispatch": round(w_dec, 1),
        "dispatches": [nf, nw],
        "copy_bytes": copy_bytes,
        "copy_fetch_size_kib": round(f_cpy, 1),
        "copy_write_size_kib": round(w_cpy, 1),
        "fetch_scale": round(k_fetch, 4),
        "write_scale": round(k_write, 4),
        "hbm_read_bytes_per_launch": int(read_b),
        "hbm_write_bytes_per_launch": int(write_b),
        "hbm_bytes_per_launch": int(read_b + write_b),
        "kernel_source_hash": kernel_source_hash(),
    }
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_pmc.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def cpu_baseline(w, min_seconds=10.0, max_seconds=30.0, meta_half=False, n_out=0,
                 rope_theta=0.0):
    """The C oracle (single thread) on a bounded sample of the same workload:
    whole decode steps (append with its flush, then attention for all 256
    query heads) repeated until about `min_seconds` of CPU work."""
    import numpy as np

    import oracle
    from kv_cache_bit_kivi_amd import synth

    k, v = synth.kv(w)
    cap = w.capacity(64)
    # one oracle cache per sequence for a ragged batch, one for the whole batch otherwise
    groups = ([(b, b + 1) for b in range(w.batch)] if w.ragged else [(0, w.batch)])
    ctx, tqs = w.contexts(), w.tqs()
    ocs = []
    for b0, b1 in groups:
        oc = oracle.OracleCache(b1 - b0, w.kv_heads, w.gqa, w.head_dim, w.bits, w.group,
                                w.residual, cap, meta_half=meta_half, n_out=n_out,
                                rope_theta=rope_theta)
        oc.prefill(k[b0:b1, :, : int(ctx[b0])], v[b0:b1, :, : int(ctx[b0])], int(tqs[b0]))
        ocs.append(oc)
    del k, v
    mb = 2 if meta_half else 4
    nbytes, steps, t_total = 0, 0, 0.0
    while t_total < min_seconds and steps < 64:
        kn, vn = synth.new_token(w, steps + 1)
        q = synth.query(w, steps + 1)
        for (b0, b1), oc in zip(groups, ocs):
            flush = oc.tr == w.residual
            t0 = time.perf_counter()
            oc.append(np.ascontiguousarray(kn[b0:b1]), np.ascontiguousarray(vn[b0:b1]))
            oc.decode(np.ascontiguousarray(q[b0:b1]), w.softmax_scale)
            t_total += time.perf_counter() - t0
            n = b1 - b0
            nbytes += append_bytes(n, w.kv_heads, w.head_dim, w.bits, w.group, w.residual,
                                   flush, mb, n_out)
            nbytes += decode_bytes(n, w.kv_heads, w.gqa, w.head_dim, w.bits, w.group, oc.tq,
                                   oc.tr, mb, n_out)
        steps += 1
        if t_total > max_seconds:
            break
    return {
        "value": round(nbytes / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{steps} whole decode steps of the same workload (one layer: append incl. "
                  f"flush, then attention for all {w.batch * w.q_heads} query heads), "
                  f"{t_total:.1f} s single-threaded",
        "seconds_per_step": round(t_total / steps, 4),
        "query_heads_per_s": round(steps * w.batch * w.q_heads / t_total, 2),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="timed steps (default: 128 per rotated layer cache)")
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="llama2_7b_b8_ctx4096")
    ap.add_argument("--layers", type=int, default=0,
                    help="layer caches the steps rotate over (default: 32, Llama-2-7B's layer "
                         "count, or fewer so that they stay within 16 GB)")
    ap.add_argument("--splits", type=int, default=0, help="decode split count (0 = automatic)")
    ap.add_argument("--meta", choices=["fp32", "fp16"], default="fp32",
                    help="storage of the quantization scales and zeros")
    ap.add_argument("--bits", type=int, default=0, choices=[0, 1, 2, 3, 4],
                    help="code width (0: the workload's own)")
    ap.add_argument("--outliers", type=int, default=0, metavar="N",
                    help="isolate N key outliers per key group (dense-and-sparse keys)")
    ap.add_argument("--key-spikes", type=float, default=None, metavar="P",
                    help="fraction of key entries multiplied by 20 (default: 0.01 with "
                         "--outliers, else 0)")
    ap.add_argument("--rope", type=float, default=0.0, metavar="THETA",
                    help="pre-RoPE keys: decode applies the rotary embedding with base THETA "
                         "(Llama-2: 10000) at each key's position")
    ap.add_argument("--paged", type=int, default=0, metavar="P",
                    help="paged quantized store with P-token pages (0: contiguous planes); the "
                         "block table is a seeded shuffle of the page pool")
    ap.add_argument("--deterministic", action="store_true",
                    help="deterministic caches: every decode wave keeps a fixed run of tiles "
                         "(repeatable bits) instead of sharing the block's tiles")
    ap.add_argument("--separate", action="store_true",
                    help="kivi_append then kivi_decode_attn (two calls) instead of the fused call")
    ap.add_argument("--window", type=int, default=16, metavar="W",
                    help="HIP events bracket windows of W consecutive timed steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB (PMC calibration)")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_MIB", "CMD"),
                    help="write the calibrated traffic summary from two PMC runs and exit")
    args = ap.parse_args()

    meta_half = args.meta == "fp16"
    mb = 2 if meta_half else 4
    # profiles are keyed by workload and metadata width
    n_out = args.outliers
    rope = float(args.rope)
    tag = (args.workload + (f"_b{args.bits}" if args.bits else "") +
           (f"_out{n_out}" if n_out else "") + ("_rope" if rope > 0 else "") +
           (f"_paged{args.paged}" if args.paged else "") + ("_meta16" if meta_half else "") +
           ("_det" if args.deterministic else ""))
    if args.pmc_summary:
        fcsv, wcsv, mib, cmd = args.pmc_summary
        pmc_summary(fcsv, wcsv, int(mib) << 20, tag, cmd)
        return

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the kernels shard across GPUs by (batch, KV head) with no exchange, but this "
              "build measures one GPU only).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from kv_cache_bit_kivi_amd import synth
    from kv_cache_bit_kivi_amd._lib import lib
    from kv_cache_bit_kivi_amd.cache import KiviCache, PagedKiviCache, RaggedKiviCache

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    lib()  # fails loudly if the HIP library is missing
    torch.cuda.set_device(0)
    w = synth.WORKLOADS[args.workload]
    if args.bits:
        w = w.with_(bits=args.bits)
    spikes = args.key_spikes if args.key_spikes is not None else (0.01 if n_out else 0.0)
    if spikes:
        w = w.with_(key_spikes=spikes)
    B, H, r, D, bits, G, R = (w.batch, w.kv_heads, w.gqa, w.head_dim, w.bits, w.group,
                              w.residual)
    if args.layers <= 0:
        layer_bytes = decode_bytes(B, H, r, D, bits, G, int(w.context), R, mb, n_out)
        args.layers = int(max(2, min(32, 16e9 // layer_bytes)))
    if args.steps <= 0:
        args.steps = 128 * args.layers
    NL = args.layers
    total_steps = args.warmup + args.steps
    per_layer_appends = (total_steps + NL - 1) // NL
    cap = w.capacity(per_layer_appends + R)

    paged = args.paged > 0
    ragged = w.ragged or paged      # (the paged calls carry per-sequence lengths)
    ctx0 = w.contexts().astype(np.int32)          # per-sequence lengths at the start
    tq0 = w.tqs().astype(np.int32)
    tr0 = ctx0 - tq0
    k, v = synth.kv(w)
    kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    del k, v
    caches = []
    if paged:
        cap = (cap + args.paged - 1) // args.paged * args.paged
    for li in range(NL):
        if paged:
            mp = cap // args.paged
            perm = np.random.default_rng(1000 + li).permutation(B * mp).astype(np.int32)
            c = PagedKiviCache(B, H, r, D, bits, G, R, cap, args.paged, num_pages=B * mp,
                               table=perm.reshape(B, mp), meta_half=meta_half, outliers=n_out,
                               rope_theta=rope, deterministic=args.deterministic)
            c.prefill(kd, vd, ctx0, tq0)
        elif ragged:
            c = RaggedKiviCache(B, H, r, D, bits, G, R, cap, meta_half=meta_half,
                                outliers=n_out, rope_theta=rope,
                                deterministic=args.deterministic)
            c.prefill(kd, vd, ctx0, tq0)
        else:
            c = KiviCache(B, H, r, D, bits, G, R, cap, meta_half=meta_half, outliers=n_out,
                          rope_theta=rope, deterministic=args.deterministic)
            c.prefill(kd, vd, w.tq)
        caches.append(c)
    del kd, vd
    # distinct synthetic tokens / queries for every step, resident on the GPU
    n_tok = min(total_steps, 256)
    knew, vnew, qs = [], [], []
    for s in range(n_tok):
        kn, vn = synth.new_token(w, s + 1)
        knew.append(torch.from_numpy(kn).cuda())
        vnew.append(torch.from_numpy(vn).cuda())
        qs.append(torch.from_numpy(synth.query(w, s + 1)).cuda())
    outs = [torch.empty((B, H * r, D), dtype=torch.float16, device="cuda") for _ in range(NL)]
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(4):
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    for c in caches:
        c.workspace_for(args.splits)
    torch.cuda.synchronize()

    # The step loop calls the C ABI directly with pointers bound once, so the
    # host enqueues faster than the GPU drains and the events bracket queued
    # work, not host-side gaps.
    import ctypes

    L = lib()
    cur = torch.cuda.current_stream()
    stream = cur.cuda_stream
    kptr = [t.data_ptr() for t in knew]
    vptr = [t.data_ptr() for t in vnew]
    qptr = [t.data_ptr() for t in qs]
    optr = [t.data_ptr() for t in outs]
    wsp = [(c.workspace.data_ptr(), c.workspace.numel()) if c.workspace is not None else (None, 0)
           for c in caches]
    scale = float(w.softmax_scale)
    if paged:
        crefs = [ctypes.byref(c.pc) for c in caches]
        append_fn, decode_fn = L.kivi_paged_append, L.kivi_paged_decode_attn
        fused_fn = L.kivi_paged_append_decode_attn
    elif ragged:
        crefs = [ctypes.byref(c.rc) for c in caches]
        append_fn, decode_fn = L.kivi_ragged_append, L.kivi_ragged_decode_attn
        fused_fn = L.kivi_ragged_append_decode_attn
    if ragged:

        def flushes(li):          # sequences whose residual is full (flush on this append)
            return caches[li].tr_arr == R

        def lengths(li):
            return caches[li].tq_arr.copy(), caches[li].tr_arr.copy()
    else:
        crefs = [ctypes.byref(c.c) for c in caches]
        append_fn, decode_fn = L.kivi_append, L.kivi_decode_attn
        fused_fn = L.kivi_append_decode_attn

        def flushes(li):
            return caches[li].c.tr == R

        def lengths(li):
            return caches[li].c.tq, caches[li].c.tr

    def step(i):
        li = i % NL
        j = i % n_tok
        fl = flushes(li)
        if args.separate:
            rc = append_fn(crefs[li], kptr[j], vptr[j], stream)
            if rc:
                raise RuntimeError(f"append failed: {rc}")
            rc = decode_fn(crefs[li], qptr[j], scale, optr[li], wsp[li][0], wsp[li][1],
                           args.splits, stream)
        else:
            rc = fused_fn(crefs[li], kptr[j], vptr[j], qptr[j], scale, optr[li], wsp[li][0],
                          wsp[li][1], args.splits, stream)
        if rc:
            raise RuntimeError(f"decode step failed: {rc}")
        return (fl, *lengths(li))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    for c in caches:       # back to the workload's starting lengths
        if ragged:
            c.set_lengths(tq0, tr0)
        else:
            c.set_lengths(w.tq, w.tr)
    splits_used = caches[0].auto_splits() if args.splits == 0 else args.splits

    # HIP events on the launch stream bracket windows of up to W consecutive
    # steps that flush nothing (an event is a packet on that stream:
    # bracketing every launch would add its own dispatch latency to each
    # measured launch and slow the loop).  Whether a step flushes is known on
    # the host before its call, so a window closes before any flush step.
    W = max(1, args.window)
    pool = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps + 2)]
    windows, open_w, pi = [], None, 0
    meta = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        fl = bool(np.any(flushes(i % NL)))
        if open_w is not None and (fl or len(open_w[2]) == W):
            open_w[1].record(cur)
            windows.append(open_w)
            open_w = None
        if not fl and open_w is None:
            open_w = (pool[pi], pool[pi + 1], [])
            pi += 2
            open_w[0].record(cur)
        meta.append(step(i))
        if open_w is not None:
            open_w[2].append(i)
    if open_w is not None:
        open_w[1].record(cur)
        windows.append(open_w)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # algorithmic bytes of every step, at the lengths the decode reads (after
    # the step's append); ragged: summed over the sequences
    per_seq = 1 if ragged else B
    dec_bytes = [int(np.sum(decode_bytes(per_seq, H, r, D, bits, G, np.asarray(tq, np.int64),
                                         np.asarray(tr, np.int64), mb, n_out)))
                 for _, tq, tr in meta]
    app_bytes = [int(np.sum([append_bytes(per_seq, H, D, bits, G, R, bool(f), mb, n_out)
                             for f in np.atleast_1d(fl)]))
                 for fl, _, _ in meta]
    total_bytes = sum(dec_bytes) + sum(app_bytes)
    # The timed call is the decode launch, carrying the new token's append when
    # fused (separate mode: the append launch too); windows hold no flush.
    new_tok = append_bytes(B, H, D, bits, G, R, False, mb, n_out)
    per_call = [d + new_tok for d in dec_bytes]
    win_ms = np.array([e0.elapsed_time(e1) / len(ix) for e0, e1, ix in windows])
    win_bytes = np.array([sum(per_call[i] for i in ix) / len(ix) for _, _, ix in windows])
    if not len(win_ms):
        raise SystemExit("every timed step flushes: raise --steps")
    n_launch = sum(len(ix) for _, _, ix in windows)
    w_time = float(sum(t * len(ix) for t, (_, _, ix) in zip(win_ms, windows)))   # ms
    w_bytes = float(sum(b * len(ix) for b, (_, _, ix) in zip(win_bytes, windows)))
    n_flush = sum(int(np.sum(fl)) for fl, _, _ in meta)

    value = total_bytes / elapsed / 1e9
    achieved = w_bytes / (w_time * 1e-3) / 1e9
    if ragged:
        kind = "paged" if paged else "ragged"
        calls = (f"kivi_{kind}_append + kivi_{kind}_decode_attn" if args.separate
                 else f"kivi_{kind}_append_decode_attn")
    else:
        calls = "kivi_append + kivi_decode_attn" if args.separate else "kivi_append_decode_attn"

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": B, "q_heads": H * r, "kv_heads": H, "head_dim": D,
            "context_at_start": (w.context if not ragged else
                                 {"min": int(ctx0.min()), "mean": round(float(ctx0.mean()), 1),
                                  "max": int(ctx0.max()), "per_sequence": ctx0.tolist()}),
            "bits": bits, "group": G, "residual": R,
            "scale_zero": "fp16" if meta_half else "fp32",
            "key_outliers_per_group": n_out,
            "pre_rope_keys_theta": rope,
            "decode_tiles": ("fixed per-wave runs (deterministic)" if args.deterministic
                             else "shared by a block's waves in load-return order"),
            "key_spikes": w.key_spikes,
            "store": f"paged, {args.paged}-token pages, shuffled block table" if paged
                     else "contiguous planes",
            "layers_rotated": NL, "decode_splits": splits_used,
            "step_call": calls,
            "sequence_flushes_in_timed_region": n_flush,
        },
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "query_heads_per_s": round(args.steps * B * H * r / elapsed, 1),
        "roofline": {
            "bound": "hbm",
            "kernel": (f"{calls} (append and decode launches)" if args.separate
                       else f"kivi decode attention with the append folded in ({calls}: one "
                       "decode launch per step)") +
                      f"; HIP events around runs of up to {W} consecutive steps without a flush",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(tag),
            "bytes_per_launch": int(w_bytes / n_launch),
            "launches_averaged": int(n_launch),
            "window_launches": W,
            "windows": len(windows),
            "avg_launch_us": round(w_time / n_launch * 1e3, 3),
            "window_p10_us": round(float(np.percentile(win_ms, 10)) * 1e3, 3),
            "window_p90_us": round(float(np.percentile(win_ms, 90)) * 1e3, 3),
        },
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, meta_half=meta_half,
                                              n_out=n_out, rope_theta=rope)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the quantized-KV decode hot path on one MI355X.

A step is one decode step of one attention layer of the Llama-2-7B-shaped
workload (batch 8, 32 heads, head_dim 128, 2-bit codes, G = 32, R = 128):
append the new token's K/V (quantizing the full residual into the grouped
part first when it is full), then decode attention for every query head, as
one kivi_append_decode_attn call (the append is folded into the decode
launch; `--separate` times kivi_append + kivi_decode_attn instead).

Steps rotate over `--layers` independent layer caches, by default the
model's 32 layers (4.6 GB in total; fewer for larger layers, within 16 GB),
as a decode step of the whole model visits them, so that no step finds its
cache resident in the 256 MB Infinity Cache left by the previous step.  Each
layer cache starts one token short of the workload's context (3968 quantized
+ 127 residual tokens), so a layer's first step decodes exactly the
workload's call (3968 + 128 tokens); every later visit appends one more
token and the full residual is flushed once per 128 visits of a layer, the
method's own rate (streaming workloads start at their prefill instead).

Prints one JSON line: whole-step algorithmic HBM GB/s (value), query-heads/s,
the roofline of the dominant kernel (decode attention with the folded append,
timed with HIP events on the launch stream around windows of up to
`--window` consecutive calls inside the timed region; windows of steps that
flush are timed apart and reported under `flush_steps`), the codec's
throughput on the layer prefills, and the CPU oracle timed on a bounded
sample, on one core and on the host's cores.
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
# GPU work before the timed region: at least this many steps, whatever
# --warmup says, so that every layer cache (32 by default) has been visited
# many times, its first flush included, before the timed region.  A burst of
# flushes (codec launches) slows the decode launches that follow it by up to
# 15% for a few hundred launches while the shader clock recovers (kernel
# traces of the batch-8 Llama and Mistral-shaped runs); the warm-up ends
# about 2000 launches after its burst, so a short timed region sees the
# steady clock that most launches of a long run see.
MIN_WARMUP_STEPS = 2048
LAT_REPS = 64
LAT_SPIN_CYCLES = 2_000_000
PF_SPIN_CYCLES = 20_000_000
# worker processes of the multi-core CPU leg: the host's cores, at most 16
MAX_CPU_WORKERS = 16


def decode_bytes(B, H, r, D, bits, G, tq, tr, mb=4, n_out=0, v_window=False, R=0):
    """Algorithmic bytes of one decode call: packed K/V codes, scale and zero
    of both (mb bytes each: 4 for binary32, 2 for binary16), the key-outlier
    words (n_out 4-byte words per key group and channel), fp16 residual K/V,
    fp16 q and out.  With the value window the values are quantized up to
    max(0, tq + tr - R) and the rest are read from the fp16 window."""
    import numpy as np
    tv = np.maximum(tq + tr - R, 0) if v_window else tq
    per = (tq * D * bits // 8 + tv * D * bits // 8 + (tq // G) * D * 2 * mb
           + tv * (D // G) * 2 * mb + (tq // G) * n_out * D * 4 + 2 * tr * D
           + 2 * (tq + tr - tv) * D + 4 * r * D)
    return B * H * per


def append_bytes(B, H, D, bits, G, R, flush, mb=4, n_out=0, v_window=False, v_leave=False):
    """Algorithmic bytes of one append: read the new K/V token, write it to
    the residual; a flush reads R residual tokens of K and V and writes their
    codes, scales, zeros and key-outlier words.  With the value window a
    flush covers the keys only, and a value leaving the window (v_leave) is
    read from it and written as codes, scales and zeros."""
    b = B * H * D * 2 * 2 * 2
    if flush and not v_window:
        b += B * H * (2 * R * D * 2 + 2 * R * D * bits // 8 + (R // G) * D * 2 * mb
                      + R * (D // G) * 2 * mb + (R // G) * n_out * D * 4)
    if flush and v_window:
        b += B * H * (R * D * 2 + R * D * bits // 8 + (R // G) * D * 2 * mb
                      + (R // G) * n_out * D * 4)
    if v_window and v_leave:
        b += B * H * (D * 2 + D * bits // 8 + (D // G) * 2 * mb)
    return b


def prefill_bytes(H, D, bits, G, tq, tr, mb=4, n_out=0, v_window=False, R=0):
    """Algorithmic bytes of a prefill, summed over sequences (tq, tr: arrays
    or ints per sequence): read tq fp16 tokens of K and V and write their
    codes, scales, zeros and outlier words; copy tr fp16 tokens of K and V
    into the residual (read and write).  With the value window the values
    are quantized up to max(0, tq + tr - R) and the rest copied."""
    import numpy as np
    tq = np.asarray(tq, np.int64)
    tr = np.asarray(tr, np.int64)
    tv = np.maximum(tq + tr - R, 0) if v_window else tq
    per = (tq * D * 2 + tq * D * bits // 8 + (tq // G) * D * 2 * mb
           + (tq // G) * n_out * D * 4 + tr * D * 2 * 2
           + tv * D * 2 + tv * D * bits // 8 + tv * (D // G) * 2 * mb
           + (tq + tr - tv) * D * 2 * 2)
    return int(H * np.sum(per))


def plan_steps(steps, layers, tq_start, tr_start, R, window):
    """Host replay of the cache lengths over the timed steps.

    Step i visits layer i % layers; each layer starts at (tq_start, tr_start)
    (ints, or per-sequence arrays for ragged batches) and every step appends
    one token per sequence with the lazy flush of the library: a sequence
    whose residual holds R tokens is quantized into the grouped part first.

    Returns (steps_info, windows).  steps_info[i] = (layer, flush, tq, tr):
    the sequences that flush at step i (bool array) and the lengths the
    step's decode reads.  windows: runs of consecutive steps of one kind
    (flushing or not), at most `window` steps each, as (flushes, [steps]);
    together they cover every step exactly once, in order.
    """
    import numpy as np
    if steps < 1 or layers < 1 or window < 1:
        raise ValueError("steps, layers and window must be positive")
    tq0 = np.atleast_1d(np.asarray(tq_start, np.int64))
    tr0 = np.atleast_1d(np.asarray(tr_start, np.int64))
    if np.any(tr0 < 0) or np.any(tr0 > R):
        raise ValueError("residual length outside [0, R]")
    tqs = [tq0.copy() for _ in range(layers)]
    trs = [tr0.copy() for _ in range(layers)]
    info = []
    for i in range(steps):
        li = i % layers
        fl = trs[li] == R
        tqs[li] = tqs[li] + np.where(fl, R, 0)
        trs[li] = np.where(fl, 0, trs[li]) + 1
        info.append((li, fl, tqs[li].copy(), trs[li].copy()))
    windows = []
    for i, (_, fl, _, _) in enumerate(info):
        kind = bool(np.any(fl))
        if windows and windows[-1][0] == kind and len(windows[-1][1]) < window:
            windows[-1][1].append(i)
        else:
            windows.append((kind, [i]))
    return info, windows


# timed steps left out of the roofline windows at the start of the timed
# region (see timed_windows' caller)
LEAD_STEPS = 2


def timed_windows(windows, lead):
    """The windows of plan_steps without the first `lead` steps, as long as a
    window remains (a run of at most `lead` steps keeps its last step)."""
    windows = [(fl, list(ix)) for fl, ix in windows]
    for _ in range(lead):
        if len(windows[0][1]) > 1:
            windows[0] = (windows[0][0], windows[0][1][1:])
        elif len(windows) > 1:
            windows = windows[1:]
    return windows


def start_lengths(w):
    """(tq, tr) arrays every layer cache starts the timed steps at: one token
    short of the workload's context, so the first step decodes the
    workload's own call; a streaming workload starts at its prefill; a cache
    with an empty residual (everything quantized) starts as it is."""
    import numpy as np
    tq = w.tqs().astype(np.int64)
    tr = w.contexts().astype(np.int64) - tq
    if w.steps == 0:
        tr = np.where(tr > 0, tr - 1, tr)
    return tq, tr


DECODE_SOURCES = ("decode_mfma_impl.h", "decode_mfma.hip", "decode_mfma_ragged.hip",
                  "decode_mfma_paged.hip", "decode_mfma_o1.hip", "decode_mfma_o2.hip",
                  "decode_mfma_ragged_o.hip", "decode_mfma_paged_o.hip", "decode_mfma_rope.hip",
                  "decode_mfma_ragged_rope.hip", "decode_mfma_paged_rope.hip", "kivi_internal.h",
                  "kivi_api.hip")


def kernel_source_hash() -> str:
    """Hash of the sources that define the decode kernel and its launch, and
    of the build script (its per-source compiler flags)."""
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        h.update(name.encode())
        h.update(open(os.path.join(ROOT, "kv_cache_bit_kivi_amd", "csrc", name), "rb").read())
    h.update(open(os.path.join(ROOT, "kv_cache_bit_kivi_amd", "build.py"), "rb").read())
    return h.hexdigest()[:16]


DECODE_KERNEL = "decode_mfma_kernel"
# PMC calibration kernel: torch's elementwise bitwise_not over N bytes, a plain
# copy-shaped kernel (reads N bytes, writes N bytes) with a recognisable name
COPY_KERNEL_HINT = "bitwise_not"


def measured_traffic(workload: str):
    """(HBM bytes per decode launch, their ratio to the algorithmic bytes of
    the same dispatches) from the committed rocprofv3 PMC summary, only if it
    was taken on the current kernel sources; else (None, None).  The PMC run
    is the workload's default run (warm-up and timed steps), so its launches
    read at their own lengths: the ratio, not the byte count, carries over to
    another run of the workload."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_pmc.json")
    if not os.path.exists(path):
        return None, None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None, None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None, None
    return d.get("hbm_bytes_per_launch"), d.get("traffic_over_algorithmic")


def pmc_summary(fetch_csv: str, write_csv: str, copy_bytes: int, workload: str, command: str,
                alg_mean: float, alg_dispatches: int):
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
        # the algorithmic bytes of the same dispatches (warm-up and timed
        # steps, at the lengths each one read), for the comparison
        "algorithmic_bytes_per_dispatch": int(alg_mean),
        "algorithmic_dispatches": alg_dispatches,
        "traffic_over_algorithmic": round((read_b + write_b) / alg_mean, 4),
        "kernel_source_hash": kernel_source_hash(),
    }
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_pmc.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


# ---------------------------------------------------------------- CPU leg

def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_units(w, units, steps, kw):
    """The oracle on (batch, KV-head) units, each a one-sequence, one-head
    cache: prefill (not timed), then `steps` whole decode steps (append with
    its flush, then attention for the unit's query heads).  Returns (start,
    end, bytes, steps) with perf_counter times (system-wide monotonic)."""
    import numpy as np

    import oracle
    from kv_cache_bit_kivi_amd import synth

    r = w.gqa
    ctx, tqs = w.contexts(), w.tqs()
    tq_s, tr_s = start_lengths(w)
    cap = w.capacity(steps + 64)
    caches = []
    for b, h in units:
        L = int(ctx[b])
        k = synth.k_plane(w, b, h, L)[None, None]
        v = synth.v_plane(w, b, h, L)[None, None]
        oc = oracle.OracleCache(1, 1, r, w.head_dim, w.bits, w.group, w.residual, cap, **kw)
        oc.prefill(k, v, int(tqs[b]))
        oc.tq, oc.tr = int(tq_s[b]), int(tr_s[b])
        caches.append(oc)
    # the step's inputs are generated before its timed part
    mb = 2 if kw.get("meta_half") else 4
    n_out = kw.get("n_out", 0)
    t_busy, nbytes = 0.0, 0
    t0 = time.perf_counter()
    for s in range(1, steps + 1):
        kn, vn = synth.new_token(w, s)
        q = synth.query(w, s)
        ins = [(np.ascontiguousarray(kn[b:b + 1, h:h + 1]), np.ascontiguousarray(vn[b:b + 1, h:h + 1]),
                np.ascontiguousarray(q[b:b + 1, h * r:(h + 1) * r])) for b, h in units]
        t1 = time.perf_counter()
        vw = bool(kw.get("v_window"))
        for oc, (kk, vv, qq) in zip(caches, ins):
            flush = oc.tr == w.residual
            leave = oc.tq + oc.tr >= w.residual
            oc.append(kk, vv)
            oc.decode(qq, w.softmax_scale)
            nbytes += append_bytes(1, 1, w.head_dim, w.bits, w.group, w.residual, flush, mb,
                                   n_out, vw, leave)
            nbytes += int(decode_bytes(1, 1, r, w.head_dim, w.bits, w.group, oc.tq, oc.tr, mb,
                                       n_out, vw, w.residual))
        t_busy += time.perf_counter() - t1
    return t0, time.perf_counter(), t_busy, nbytes


def _cpu_worker(args):
    w, units, steps, kw = args
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    return _cpu_units(w, units, steps, kw)


def cpu_baseline(w, min_seconds=10.0, max_seconds=30.0, meta_half=False, n_out=0,
                 rope_theta=0.0, workers=None, pool=None, v_window=False):
    """The C oracle (single-threaded code) on a bounded sample of the same
    workload: whole decode steps over every (batch, KV-head) unit.

    One core: the units run in this process, step after step, until about
    `min_seconds` of oracle time.  Host cores: the same units fanned out over
    `workers` processes (default: the host's cores, at most 16), each running
    the single-threaded oracle on its share for the same kind of steps; the
    rate is the bytes of all units over the wall time from the first start to
    the last finish."""
    kw = dict(meta_half=meta_half, n_out=n_out, rope_theta=rope_theta)
    if v_window:
        kw["v_window"] = True
    units = [(b, h) for b in range(w.batch) for h in range(w.kv_heads)]
    # one core: grow the step count until the sample is long enough
    steps, spent = 1, 0.0
    while True:
        _, _, busy, nbytes = _cpu_units(w, units, steps, kw)
        spent += busy
        if busy >= min_seconds or steps >= 64 or spent > max_seconds:
            break
        steps = min(64, max(steps + 1, int(steps * min_seconds / max(busy, 1e-3)) + 1))
    one = {"value": round(nbytes / busy / 1e9, 4), "seconds_per_step": round(busy / steps, 4),
           "steps": steps, "query_heads_per_s": round(steps * w.batch * w.q_heads / busy, 2)}
    res = {
        "value": one["value"],
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{steps} whole decode steps of the same workload (one layer: append incl. "
                  f"flush, then attention for all {w.batch * w.q_heads} query heads), "
                  f"{busy:.1f} s single-threaded",
        "one_core": one,
        "cpu_model": cpu_model(),
        "host_cores_visible": len(os.sched_getaffinity(0)),
    }
    n = workers if workers is not None else min(len(os.sched_getaffinity(0)), MAX_CPU_WORKERS)
    n = max(1, min(n, len(units)))
    if n > 1:
        # as many steps as fit about min_seconds on n cores
        msteps = int(min(256, max(steps, min_seconds * n / max(one["seconds_per_step"], 1e-6))))
        shares = [units[i::n] for i in range(n)]
        jobs = [(w, s, msteps, kw) for s in shares]
        if pool is not None:
            outs = pool.map(_cpu_worker, jobs)
        else:
            import multiprocessing as mp
            with mp.get_context("fork").Pool(n) as p:
                outs = p.map(_cpu_worker, jobs)
        # timed part of each worker: its steps, after its own prefill
        t_first = min(o[1] - o[2] for o in outs)
        t_last = max(o[1] for o in outs)
        wall = t_last - t_first
        nb = sum(o[3] for o in outs)
        res.update({
            "value": round(nb / wall / 1e9, 4),
            "cores": n,
            "sample": f"{msteps} whole decode steps of the same workload (one layer: append "
                      f"incl. flush, then attention for all {w.batch * w.q_heads} query heads), "
                      f"its {len(units)} (batch, KV-head) units over {n} processes, "
                      f"{wall:.1f} s wall; one core: {steps} steps, {busy:.1f} s",
            "seconds_per_step": round(wall / msteps, 4),
            "query_heads_per_s": round(msteps * w.batch * w.q_heads / wall, 2),
        })
    else:
        res.update({"seconds_per_step": one["seconds_per_step"],
                    "query_heads_per_s": one["query_heads_per_s"]})
    return res


# ---------------------------------------------------------------- GPU leg

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="timed steps (default: 128 per rotated layer cache; streaming "
                         "workloads: their own step count per layer)")
    ap.add_argument("--warmup", type=int, default=64,
                    help=f"untimed steps before the timed region (at least {MIN_WARMUP_STEPS} "
                         "are run, see warmup_effective)")
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
    ap.add_argument("--v-window", action="store_true",
                    help="values keep a sliding window of the R newest tokens (uniform caches; "
                         "generic decode kernel)")
    ap.add_argument("--deterministic", action="store_true",
                    help="deterministic caches: every decode wave keeps a fixed run of tiles "
                         "(repeatable bits) instead of sharing the block's tiles")
    ap.add_argument("--separate", action="store_true",
                    help="kivi_append then kivi_decode_attn (two calls) instead of the fused call")
    ap.add_argument("--window", type=int, default=256, metavar="W",
                    help="HIP events bracket windows of up to W consecutive timed steps (an "
                         "event delays the next launch by several microseconds, so windows "
                         "are long)")
    ap.add_argument("--window-trace", metavar="PATH",
                    help="also write every window's (first step, steps, flushes, us per step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cpu-workers", type=int, default=None,
                    help="processes of the multi-core CPU leg (default: host cores, at most 16)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB (PMC calibration)")
    ap.add_argument("--latency-reps", type=int, default=LAT_REPS,
                    help="prefill + step pairs timed for latency_us (0: skip)")
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
           ("_det" if args.deterministic else "") + ("_vwin" if args.v_window else ""))
    if args.gpus != 1 and not args.pmc_summary:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the kernels shard across GPUs by (batch, KV head) with no exchange, but this "
              "build measures one GPU only).", file=sys.stderr)
        sys.exit(2)
    if args.steps < 0 or args.warmup < 0:
        print("--steps and --warmup must not be negative", file=sys.stderr)
        sys.exit(2)

    import numpy as np

    from kv_cache_bit_kivi_amd import synth

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
    NL = args.layers
    if args.steps == 0:
        args.steps = (w.steps or 128) * NL
    warm = max(args.warmup, MIN_WARMUP_STEPS)
    tq_s, tr_s = start_lengths(w)
    paged = args.paged > 0
    ragged = w.ragged or paged      # (the paged calls carry per-sequence lengths)
    W = max(1, args.window)
    per_seq = 1 if ragged else B
    vw = args.v_window

    def dec_bytes_of(info):
        # algorithmic bytes of each planned step's decode, at the lengths it
        # reads (after the step's append); ragged: summed over the sequences
        return [int(np.sum(decode_bytes(per_seq, H, r, D, bits, G, tq, tr, mb, n_out, vw, R)))
                for _, _, tq, tr in info]

    if args.pmc_summary:
        # the counters average every decode dispatch of the profiled run: the
        # warm-up's and the timed steps' (no latency pairs in PMC runs), each
        # with the new token folded in
        new_tok = append_bytes(B, H, D, bits, G, R, False, mb, n_out)
        plans = [plan_steps(n, NL, tq_s if ragged else tq_s[:1], tr_s if ragged else tr_s[:1],
                            R, W)[0] for n in (warm, args.steps)]
        allb = [d + new_tok for info in plans for d in dec_bytes_of(info)]
        fcsv, wcsv, mib, cmd = args.pmc_summary
        pmc_summary(fcsv, wcsv, int(mib) << 20, tag, cmd, sum(allb) / len(allb), len(allb))
        return

    # The multi-core CPU leg's worker processes are forked now, before this
    # process touches the GPU, and wait for their work until the GPU leg ends.
    pool = None
    n_workers = (args.cpu_workers if args.cpu_workers is not None
                 else min(len(os.sched_getaffinity(0)), MAX_CPU_WORKERS))
    if not args.no_cpu_baseline and n_workers > 1:
        import multiprocessing as mp
        pool = mp.get_context("fork").Pool(n_workers)

    import torch

    from kv_cache_bit_kivi_amd._lib import lib
    from kv_cache_bit_kivi_amd.cache import KiviCache, PagedKiviCache, RaggedKiviCache

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    lib()  # fails loudly if the HIP library is missing
    torch.cuda.set_device(0)
    # capacity for every flush of the warm-up or of the timed steps (the
    # lengths are set back to the start after the warm-up)
    per_layer = (max(warm, args.steps) + NL - 1) // NL
    cap = w.capacity(per_layer + R)

    if args.v_window and ragged:
        print("--v-window needs a uniform workload (ragged and paged caches refuse it)",
              file=sys.stderr)
        sys.exit(2)
    ctx0 = w.contexts().astype(np.int32)          # per-sequence lengths at the prefill
    tq0 = w.tqs().astype(np.int32)
    k, v = synth.kv(w)
    kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    del k, v
    caches = []
    if paged:
        cap = (cap + args.paged - 1) // args.paged * args.paged
    # each layer's prefill is timed with events: the codec's throughput.  A
    # spin kernel first, so the layers' allocations and prefills queue up
    # behind it and each event pair brackets device work, not host calls.
    cur = torch.cuda.current_stream()
    pf_ev = []
    torch.cuda._sleep(PF_SPIN_CYCLES)
    for li in range(NL):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if paged:
            mp_ = cap // args.paged
            perm = np.random.default_rng(1000 + li).permutation(B * mp_).astype(np.int32)
            c = PagedKiviCache(B, H, r, D, bits, G, R, cap, args.paged, num_pages=B * mp_,
                               table=perm.reshape(B, mp_), meta_half=meta_half, outliers=n_out,
                               rope_theta=rope, deterministic=args.deterministic)
            e0.record(cur)
            c.prefill(kd, vd, ctx0, tq0)
        elif ragged:
            c = RaggedKiviCache(B, H, r, D, bits, G, R, cap, meta_half=meta_half,
                                outliers=n_out, rope_theta=rope,
                                deterministic=args.deterministic)
            e0.record(cur)
            c.prefill(kd, vd, ctx0, tq0)
        else:
            c = KiviCache(B, H, r, D, bits, G, R, cap, meta_half=meta_half, outliers=n_out,
                          rope_theta=rope, deterministic=args.deterministic,
                          v_window=args.v_window)
            e0.record(cur)
            c.prefill(kd, vd, w.tq)
        e1.record(cur)
        pf_ev.append((e0, e1))
        caches.append(c)
    # distinct synthetic tokens / queries for every step, resident on the GPU
    n_tok = min(max(warm, args.steps), 256)
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
    pf_us = np.array([a.elapsed_time(b) * 1e3 for a, b in pf_ev])

    # The step loop calls the C ABI directly with pointers bound once, so the
    # host enqueues faster than the GPU drains and the events bracket queued
    # work, not host-side gaps.
    import ctypes

    L = lib()
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
    else:
        crefs = [ctypes.byref(c.c) for c in caches]
        append_fn, decode_fn = L.kivi_append, L.kivi_decode_attn
        fused_fn = L.kivi_append_decode_attn

    def lengths(li):
        if ragged:
            return caches[li].tq_arr.astype(np.int64), caches[li].tr_arr.astype(np.int64)
        return np.array([caches[li].c.tq], np.int64), np.array([caches[li].c.tr], np.int64)

    def set_start():
        for c in caches:
            if ragged:
                c.set_lengths(tq_s, tr_s)
            else:
                c.set_lengths(int(tq_s[0]), int(tr_s[0]))

    def step(i):
        li = i % NL
        j = i % n_tok
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

    set_start()
    for i in range(warm):
        step(i)
    # The host's bookkeeping for the timed region is done while the warm-up
    # still runs, so that the device idles only for the synchronisation
    # before the timed region (host lengths go back to the start now: every
    # warm-up launch has its lengths as launch arguments already).
    set_start()
    splits_used = caches[0].auto_splits() if args.splits == 0 else args.splits

    # HIP events on the launch stream bracket windows of up to W consecutive
    # steps of one kind (flushing or not).  An event is a packet on that
    # stream: bracketing every launch would add its own dispatch latency to
    # each measured launch and slow the loop.  Whether a step flushes is known
    # on the host before its call (plan_steps replays the lengths).
    info, windows = plan_steps(args.steps, NL, tq_s if ragged else tq_s[:1],
                               tr_s if ragged else tr_s[:1], R, W)
    # The first steps run while the host's enqueue may still trail the
    # device: the first starts on an idle queue (between an event recorded
    # before it and its kernel lies the host's enqueue latency, tens of
    # microseconds), and under the kernel tracer the launch after it waited
    # 18.6 us behind the window's start event, against 5.6 us (the event's
    # own cost) when the event follows the second step.  So the first window
    # opens after the second step's launch (it then marks that kernel's end)
    # and steps 0 and 1 stay out of the roofline (they still count in
    # `value`); a run of one or two steps keeps what it has.
    windows = timed_windows(windows, LEAD_STEPS)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in windows]
    # torch creates an event's HIP event at its first record: record each one
    # once here, so that no event is created inside the timed region (a
    # creation there held the launch after the first window event back by
    # some 80 us in a kernel trace)
    for e0, e1 in ev:
        e0.record(cur)
        e1.record(cur)
    # window k opens after the launch of the step before its first step
    opens = {ix[0] - 1: k for k, (_, ix) in enumerate(windows) if ix[0] > 0}
    closes = {ix[-1]: k for k, (_, ix) in enumerate(windows)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if windows[0][1][0] == 0:        # a one-step run: its only step is timed as it is
        ev[0][0].record(cur)
    for i in range(args.steps):
        step(i)
        k = opens.get(i)
        if k is not None:
            ev[k][0].record(cur)
        k = closes.get(i)
        if k is not None:
            ev[k][1].record(cur)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # the library's host lengths must have followed the plan
    for li in range(NL):
        last = max(i for i in range(args.steps) if i % NL == li) if args.steps > li else None
        if last is not None:
            tq_l, tr_l = lengths(li)
            assert np.array_equal(tq_l, info[last][2]) and np.array_equal(tr_l, info[last][3]), \
                "cache lengths differ from the step plan"

    # Latency of a fresh cache's first decode: a prefill of layer 0 followed by
    # one fused step, LAT_REPS pairs enqueued behind a short spin kernel so the
    # events see back-to-back device work, not the host's enqueue time; and
    # one pair timed on the host from an idle queue to its synchronisation.
    c0 = caches[0]

    def prefill0():
        if ragged:
            c0.prefill(kd, vd, ctx0, tq0)
        else:
            c0.prefill(kd, vd, w.tq)

    pair_us = host_pair_us = None
    if args.latency_reps > 0:
        for _ in range(4):
            prefill0()
            step(0)
        torch.cuda.synchronize()
        t_h = time.perf_counter()
        prefill0()
        step(0)
        torch.cuda.synchronize()
        host_pair_us = (time.perf_counter() - t_h) * 1e6
        la, lb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(LAT_SPIN_CYCLES)
        la.record(cur)
        for _ in range(args.latency_reps):
            prefill0()
            step(0)
        lb.record(cur)
        torch.cuda.synchronize()
        pair_us = la.elapsed_time(lb) * 1e3 / args.latency_reps
    del kd, vd

    # algorithmic bytes of every step, at the lengths the decode reads
    dec_bytes = dec_bytes_of(info)
    # (a value leaves the window when the cache held R tokens before the append)
    app_bytes = [int(np.sum([append_bytes(per_seq, H, D, bits, G, R, bool(f), mb, n_out, vw,
                                          bool(np.all(tq + tr - 1 >= R)))
                             for f in fl]))
                 for _, fl, tq, tr in info]
    total_bytes = sum(dec_bytes) + sum(app_bytes)
    n_flush = int(sum(int(np.sum(fl)) for _, fl, _, _ in info))
    # The dominant kernel is the decode launch, carrying the new token's
    # append when fused (separate mode: the append launch too).  With the
    # value window a step is the window append's launches and the generic
    # decode: the windows time whole steps.
    new_tok = append_bytes(B, H, D, bits, G, R, False, mb, n_out)
    per_call = ([d + a for d, a in zip(dec_bytes, app_bytes)] if vw
                else [d + new_tok for d in dec_bytes])
    win_ms = [ev[k][0].elapsed_time(ev[k][1]) for k in range(len(windows))]
    plain = [k for k, (fl, _) in enumerate(windows) if not fl]
    flushing = [k for k, (fl, _) in enumerate(windows) if fl]
    sel = plain if plain else list(range(len(windows)))
    n_launch = sum(len(windows[k][1]) for k in sel)
    w_time = float(sum(win_ms[k] for k in sel))                              # ms
    w_bytes = float(sum(per_call[i] for k in sel for i in windows[k][1]))
    per_launch_us = np.array([win_ms[k] / len(windows[k][1]) * 1e3 for k in sel])
    if args.window_trace:
        with open(args.window_trace, "w") as f:
            for k, (fl, ix) in enumerate(windows):
                f.write(f"{ix[0]} {len(ix)} {int(fl)} {win_ms[k] / len(ix) * 1e3:.3f}\n")

    value = total_bytes / elapsed / 1e9
    traffic_b, traffic_r = measured_traffic(tag)
    achieved = w_bytes / (w_time * 1e-3) / 1e9
    if ragged:
        kind = "paged" if paged else "ragged"
        calls = (f"kivi_{kind}_append + kivi_{kind}_decode_attn" if args.separate
                 else f"kivi_{kind}_append_decode_attn")
    else:
        calls = "kivi_append + kivi_decode_attn" if args.separate else "kivi_append_decode_attn"
    pf_bytes = prefill_bytes(H, D, bits, G, tq0.astype(np.int64),
                             (ctx0 - tq0).astype(np.int64), mb, n_out, vw, R)
    pf_med = float(np.median(pf_us[1:] if len(pf_us) > 1 else pf_us))

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_effective": warm,
        "ms_per_step": round(elapsed / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 io, f16/bf16 mfma (hi+lo factors), f32 acc",
        "arithmetic": ("codes, scales and zeros stored exactly (codec in IEEE binary32); fp16 "
                       "queries, residual and output; dot products on the matrix cores with the "
                       "codes as exact f16/bf16 operands and each factor split into hi + lo "
                       "halves (>= 16 significant bits), accumulated in binary32; softmax in "
                       "binary32"),
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": B, "q_heads": H * r, "kv_heads": H, "head_dim": D,
            "context_at_first_step": (int(tq_s[0] + tr_s[0] + 1) if not ragged else
                                      {"min": int((tq_s + tr_s).min() + 1),
                                       "max": int((tq_s + tr_s).max() + 1)}),
            "start_lengths_tq_tr": ([int(tq_s[0]), int(tr_s[0])] if not ragged else
                                    [tq_s.tolist(), tr_s.tolist()]),
            "bits": bits, "group": G, "residual": R,
            "scale_zero": "fp16" if meta_half else "fp32",
            "key_outliers_per_group": n_out,
            "pre_rope_keys_theta": rope,
            "value_window": bool(vw),
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
                       else f"{calls} with the value window: the window append's launches "
                       "and the generic decode kernel, timed as whole steps" if vw
                       else f"kivi decode attention with the append folded in ({calls}: one "
                       "decode launch per step)") +
                      f"; HIP events around runs of up to {W} consecutive steps (the first "
                      "two steps of the timed region left out: the host's enqueue still trails "
                      "the device there)" +
                      (" without a flush" if plain else " (every step flushes)"),
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic_b,
            "traffic_over_algorithmic": traffic_r,
            "bytes_per_launch": int(w_bytes / n_launch),
            "launches_averaged": int(n_launch),
            "window_launches": W,
            "windows": len(sel),
            "avg_launch_us": round(w_time / n_launch * 1e3, 3),
            "window_p10_us": round(float(np.percentile(per_launch_us, 10)), 3),
            "window_p90_us": round(float(np.percentile(per_launch_us, 90)), 3),
        },
        "flush_steps": ({
            "steps": int(sum(len(windows[k][1]) for k in flushing)),
            "avg_step_us": round(sum(win_ms[k] for k in flushing) * 1e3 /
                                 sum(len(windows[k][1]) for k in flushing), 3),
            "algorithmic_bytes_per_step": int(np.mean([dec_bytes[i] + app_bytes[i]
                                                       for k in flushing
                                                       for i in windows[k][1]])),
            "note": "steps whose append flushes the full residual first, timed in windows of "
                    "their own; left out of the roofline, included in value",
        } if flushing else None),
        "prefill_quantize": {
            "kernels": "kivi_prefill: quantize keys and values of the quantized part, copy the "
                       "residual (one layer)",
            "median_us": round(pf_med, 2),
            "algorithmic_bytes": pf_bytes,
            "gbps": round(pf_bytes / (pf_med * 1e-6) / 1e9, 1),
            "frac": round(pf_bytes / (pf_med * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "layers_timed": int(len(pf_us) - 1 if len(pf_us) > 1 else 1),
        },
        "kernel_source_hash": kernel_source_hash(),
    }
    # one layer's prefill (quantize the grouped part, copy the residual)
    # followed by one fused step: the latency of a fresh cache's first decode
    if pair_us is not None:
        result["latency_us"] = {
            "prefill_plus_step": round(pair_us, 2),
            "host_call_to_sync": round(host_pair_us, 2),
            "note": (f"device time of a prefill and one {calls} step on layer 0, "
                     f"{args.latency_reps} pairs back to back behind a spin kernel (host "
                     f"enqueue hidden); host_call_to_sync: one pair from an idle queue, "
                     f"host clock")}
    if w.steps:
        # streaming workloads: the layer's whole run of steps (flushes included)
        result["per_layer_run"] = {"steps": w.steps,
                                   "ms": round(elapsed * 1e3 * w.steps / args.steps, 3)}
    del caches, knew, vnew, qs, outs
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, meta_half=meta_half,
                                              n_out=n_out, rope_theta=rope,
                                              workers=n_workers, pool=pool,
                                              v_window=args.v_window)
    if pool is not None:
        pool.close()
        pool.join()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

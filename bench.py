#!/usr/bin/env python3
"""Benchmark of the paged KV-cache attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pa_paged_attention() call (cache scatter, planning, split-KV
decode, split merge, MFMA prefill) on one synthetic batch whose inputs are
already resident in HBM.  The headline workload is pure_decode: 64 single-token
decodes over 512-4096 cached tokens, 32/8 heads, head_size 128, block_size 16.
The run prints ONE JSON line on stdout; progress goes to stderr.

Timing protocol, per workload (HIP events on the library's stream):
  cold   the headline.  Before every step, outside the events, a scrub pass
         reads a 1 GiB buffer (more than the 256 MB memory-side cache plus the
         L2s), so each step starts with none of its inputs cached and with
         clean caches (a read+write scrub leaves dirty lines whose write-back
         then lands inside the timed step: pure_decode's decode measured 178
         us that way against 121 us after a read-only or a write-then-read
         scrub).  K steps, each bracketed by its own event pair; reported as
         median (ms_per_step), p10, p90 and mean.
  warm   K steps back to back with no scrub (inputs partly cached), same
         statistics, as secondary fields.
  kernel a third set of K cold steps with the library's per-kernel events
         (pa_args.kernel_events): mean and median duration of each kernel.

Reported:
  value         decode KV-read GB/s of the whole step, cold median (logical
                history bytes sum_b L_b * 2 * Hkv * D * 2 / step time)
  roofline      the dominant kernel's algorithmic bytes (or flops) per launch
                over its mean cold duration
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same
                workload, in the same unit
  also          the other workloads (mixed, long_prefill, serving, and
                pure_decode with INT8 and with INT4 caches): cold and warm step
                statistics, TFLOP/s, GB/s (serving: on unique and on logical
                history bytes; quantized caches: on code bytes), tokens/s and
                their own roofline
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode KV-read GB/s (% HBM peak); prefill TFLOP/s (% MFMA peak); tokens/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 / bf16 matrix peak
SCRUB_BYTES = 1 << 30          # cold protocol: bytes of the scrub buffer
KERNEL_SRC = {"decode": ("pa_decode.hip", "pa_elem.h", "pa_internal.h"),
              "prefill": ("pa_prefill.hip", "pa_merge.h", "pa_elem.h", "pa_internal.h"),
              "scatter_plan": ("pa_scatter.hip", "pa_internal.h")}
KERNEL_SYMBOL = {"decode": "decode_kernel", "prefill": "prefill_kernel",
                 "scatter_plan": "scatter_plan_kernel"}
TIMED = ("scatter_plan", "decode", "prefill")  # "merge" has no launch of its own


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(kernel: str) -> str:
    """Hash of the sources the kernel is built from (stale counters are ignored)."""
    h = hashlib.sha256()
    for name in KERNEL_SRC[kernel]:
        with open(os.path.join(ROOT, "paged_kv_varlen_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_means(csv_path: str, symbol: str) -> dict:
    """Mean per dispatch of each counter of the kernels whose name holds
    `symbol`, from a rocprofv3 --pmc counter_collection.csv."""
    import csv
    acc = {}
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            if symbol in row["Kernel_Name"]:
                acc.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def variant_suffix(dtype="f16", head_size=0, kv_quant="none", gate=False, prologue=0) -> str:
    """Names a workload variant in profile file names ('' for the workloads as
    defined: fp16 data and caches, their own head size, no output gate, no
    fused prologue)."""
    return ("" if dtype == "f16" else f"_{dtype}") + (f"_hd{head_size}" if head_size else "") + \
        ("" if kv_quant == "none" else f"_{kv_quant}") + ("_gate" if gate else "") + \
        (f"_rope{prologue}" if prologue else "")


VARIANT = {"suffix": ""}  # set by main() from --dtype / --head-size / --kv-quant


def write_traffic(kernel, workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv,
                  copy_bytes):
    """HBM bytes per launch of `kernel` from FETCH_SIZE / WRITE_SIZE runs (KiB per
    dispatch), each scaled by what the counter reads for a plain device copy of
    copy_bytes bytes; written to profiles/traffic_<kernel>_<workload><variant>.json."""
    sym = KERNEL_SYMBOL[kernel]
    f_k, nf = counter_means(fetch_csv, sym)["FETCH_SIZE"]
    w_k, nw = counter_means(write_csv, sym)["WRITE_SIZE"]
    f_c, _ = counter_means(copy_fetch_csv, "copyBuffer")["FETCH_SIZE"]
    w_c, _ = counter_means(copy_write_csv, "copyBuffer")["WRITE_SIZE"]
    sf, sw = copy_bytes / (f_c * 1024.0), copy_bytes / (w_c * 1024.0)
    rec = {"kernel": kernel, "workload": workload + VARIANT["suffix"],
           "source_hash": source_hash(kernel),
           "fetch_kib_per_dispatch": round(f_k, 1), "write_kib_per_dispatch": round(w_k, 1),
           "dispatches": [nf, nw], "copy_bytes": copy_bytes,
           "copy_fetch_kib": round(f_c, 1), "copy_write_kib": round(w_c, 1),
           "fetch_scale": round(sf, 4), "write_scale": round(sw, 4),
           "bytes_per_launch": int(f_k * 1024.0 * sf + w_k * 1024.0 * sw)}
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}{VARIANT['suffix']}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, or None
    when there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}{VARIANT['suffix']}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


class Runner:
    """Device copies of one batch plus the preallocated output and workspace."""

    def __init__(self, batch, torch, pa, gate=None, prologue=None):
        self.torch, self.pa, self.b = torch, pa, batch
        dev = "cuda:0"

        def to(x):  # uint16 arrays hold bf16 bit patterns
            if x is None:
                return None
            x = np.ascontiguousarray(x)
            if x.dtype == np.uint16:
                return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
            return torch.from_numpy(x).to(dev)
        self.q, self.k, self.v = to(batch.query), to(batch.key), to(batch.value)
        self.kc, self.vc = to(batch.key_cache), to(batch.value_cache)
        self.cum, self.past = to(batch.cum), to(batch.past)
        self.table, self.slots = to(batch.block_table), to(batch.slot_mapping)
        self.ks, self.vs = to(batch.k_scale), to(batch.v_scale)  # quantized caches only
        self.gate = to(gate)  # optional output gate
        self.prologue = None  # optional fused Q/K norm and rotation
        if prologue is not None:
            self.prologue = dict(prologue)
            for n in ("position_ids", "q_norm_weight", "k_norm_weight"):
                if prologue.get(n) is not None:
                    self.prologue[n] = to(prologue[n])
        D = batch.head_size
        self.out = torch.empty((batch.num_tokens, batch.num_heads * D), dtype=self.q.dtype,
                               device=dev)
        args = pa.make_args(self.q, self.k, self.v, self.kc, self.vc, self.cum, self.past,
                            self.table, self.slots, self.out, num_heads=batch.num_heads,
                            kv_num_heads=batch.kv_num_heads, scale=batch.scale,
                            k_scale=self.ks, v_scale=self.vs, gate=self.gate, prologue=self.prologue)
        self.ws = torch.empty(max(1, pa.workspace_bytes(args)), dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream()

    def step(self, events=None):
        b = self.b
        self.pa.paged_attention(self.q, self.k, self.v, self.kc, self.vc, self.cum, self.past,
                                self.table, self.slots, num_heads=b.num_heads,
                                kv_num_heads=b.kv_num_heads, scale=b.scale, output=self.out,
                                workspace=self.ws, kernel_events=events, k_scale=self.ks,
                                v_scale=self.vs, gate=self.gate, stream=self.stream,
                                prologue=self.prologue)


def stats_ms(xs) -> dict:
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 5), "p10": round(float(np.percentile(a, 10)), 5),
            "p90": round(float(np.percentile(a, 90)), 5), "mean": round(float(a.mean()), 5),
            "n": int(a.size)}


SCRUB = {"mode": "read"}


def do_scrub(scrub, torch):
    """Evict the caches: 'read' reads the 1 GiB buffer (the caches then hold
    clean, unrelated lines), 'rw' reads and writes it (dirty lines left behind
    are written back during the next step), 'flush' writes it, then reads it
    (dirty lines written back outside the events)."""
    if SCRUB["mode"] == "rw":
        scrub.add_(1)
    elif SCRUB["mode"] == "flush":
        scrub.add_(1)
        torch.sum(scrub, dtype=torch.int64)
    else:
        torch.sum(scrub, dtype=torch.int64)


def run_steps(r, steps, scrub, torch, kernel_events=False):
    """K steps, each bracketed by its own events; with a scrub tensor, a pass
    over it (do_scrub) precedes every step outside the events.  Returns
    per-step times (ms) and, with kernel_events, per-kernel times (ms) per step."""
    E = lambda: torch.cuda.Event(enable_timing=True)
    starts, ends = [E() for _ in range(steps)], [E() for _ in range(steps)]
    nk = len(r.pa.KERNELS)
    kev = [[E() for _ in range(2 * nk)] for _ in range(steps)] if kernel_events else None
    if kev is not None:
        for row in kev:  # create the underlying HIP events
            for e in row:
                e.record()
    torch.cuda.synchronize()
    for k in range(steps):
        if scrub is not None:
            do_scrub(scrub, torch)
        starts[k].record()
        r.step(None if kev is None else kev[k])
        ends[k].record()
    torch.cuda.synchronize()
    step_ms = [starts[k].elapsed_time(ends[k]) for k in range(steps)]
    if kev is None:
        return step_ms, None
    kernel_ms = {kname: [kev[s][2 * i].elapsed_time(kev[s][2 * i + 1]) for s in range(steps)]
                 for i, kname in enumerate(r.pa.KERNELS) if kname in TIMED}
    return step_ms, kernel_ms


def time_workload(name: str, steps: int, warmup: int, seed: int, torch, pa, W, scrub,
                  dtype="f16", head_size=0, kv_quant="none", gate=False, warm=True, prologue=0):
    t_gen = time.perf_counter()
    b = W.workload(name, seed, dtype=dtype, head_size=head_size, kv_quant=kv_quant)
    work = W.work(b)
    log(f"[bench] {name}: generated in {time.perf_counter() - t_gen:.1f}s "
        f"(N={b.num_tokens}, B={b.batch_size}, KV {work['kv_hist_bytes'] / 1e9:.3f} GB, "
        f"{work['flops'] / 1e12:.3f} TFLOP)")
    r = Runner(b, torch, pa, W.output_gate_input(b, seed + 1) if gate else None,
               W.prologue_inputs(b, seed + 2, rotary_dim=prologue) if prologue else None)
    for _ in range(warmup):
        r.step()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    cold, _ = run_steps(r, steps, scrub, torch)
    wall_s = time.perf_counter() - w0
    _, kernels = run_steps(r, steps, scrub, torch, kernel_events=True)
    warm_ms = run_steps(r, steps, None, torch)[0] if warm else None
    res = {"cold": stats_ms(cold), "warm": None if warm_ms is None else stats_ms(warm_ms),
           "kernel_ms": {k: stats_ms(v) for k, v in kernels.items()},
           "cold_region_wall_s": round(wall_s, 4)}
    log(f"[bench] {name}: cold median {res['cold']['median'] * 1e3:.1f} us "
        f"(p10 {res['cold']['p10'] * 1e3:.1f}, p90 {res['cold']['p90'] * 1e3:.1f})"
        + ("" if warm_ms is None else f", warm median {res['warm']['median'] * 1e3:.1f} us")
        + "; kernels (cold mean) "
        + ", ".join(f"{k} {v['mean'] * 1e3:.1f} us" for k, v in res["kernel_ms"].items()))
    del r
    torch.cuda.empty_cache()
    return b, work, res


def rates(work, ms) -> dict:
    s = ms / 1e3
    out = {"tokens_per_s": round(work["tokens"] / s, 1),
           "kv_tokens_per_s": round(work["kv_tokens"] / s, 1),
           "kv_read_GBps": round(work["kv_hist_bytes"] / s / 1e9, 2),
           "alg_TFLOPps": round(work["flops"] / s / 1e12, 3)}
    if "kv_unique_bytes" in work:
        out["kv_unique_read_GBps"] = round(work["kv_unique_bytes"] / s / 1e9, 2)
    return out


def summarize(name, work, res):
    out = {"workload": name, "ms_per_step": res["cold"]["median"], "cold": res["cold"],
           "warm": res["warm"], **rates(work, res["cold"]["median"])}
    if res["warm"] is not None:
        out["warm_rates"] = rates(work, res["warm"]["median"])
    out["kernel_us"] = {k: round(v["mean"] * 1e3, 2) for k, v in res["kernel_ms"].items()}
    out["kernel_us_median"] = {k: round(v["median"] * 1e3, 2) for k, v in res["kernel_ms"].items()}
    return out


def roofline(work, res):
    """Dominant kernel (the longer of decode and prefill, mean cold duration):
    algorithmic bytes (decode: history of the single-token rows; unique pages
    when rows share prefix pages) or flops (prefill: causally visible pairs)
    per launch over its mean duration."""
    km = res["kernel_ms"]
    dec_t, pf_t = km["decode"]["mean"] / 1e3, km["prefill"]["mean"] / 1e3
    if work["prefill_flops"] > 0 and pf_t >= dec_t:
        achieved = work["prefill_flops"] / pf_t / 1e12
        return {"kernel": "prefill", "bound": "mfma", "achieved": round(achieved, 2),
                "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic("prefill", WORKLOAD_NAME["current"]),
                "kernel_us": round(km["prefill"]["mean"] * 1e3, 2),
                "work_per_launch": work["prefill_flops"], "work_unit": "flop"}
    alg = work.get("decode_kv_unique_bytes", work["decode_kv_hist_bytes"])
    achieved = alg / dec_t / 1e9
    out = {"kernel": "decode", "bound": "hbm", "achieved": round(achieved, 1),
           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
           "traffic": measured_traffic("decode", WORKLOAD_NAME["current"]),
           "kernel_us": round(km["decode"]["mean"] * 1e3, 2), "work_per_launch": alg,
           "work_unit": "byte"}
    if "decode_kv_unique_bytes" in work:
        out["work_note"] = "unique history pages of the single-token rows (shared prefixes once)"
        out["logical_GBps"] = round(work["decode_kv_hist_bytes"] / dec_t / 1e9, 1)
    return out


WORKLOAD_NAME = {"current": ""}


def sub_batch(b, seqs, W):
    """The sequences ``seqs`` of batch b as a batch of their own (same caches)."""
    rows = np.concatenate([np.arange(b.cum[i], b.cum[i + 1]) for i in seqs]).astype(np.int64)
    pick = lambda x: None if x is None else x[rows]
    return W.Batch(name=b.name, seed=b.seed, query=b.query[rows], key=pick(b.key),
                   value=pick(b.value), key_cache=b.key_cache, value_cache=b.value_cache,
                   cum=W.cum_from_lens(b.q_lens[seqs]), past=b.past[seqs],
                   block_table=b.block_table[seqs], slot_mapping=pick(b.slot_mapping),
                   num_heads=b.num_heads, kv_num_heads=b.kv_num_heads, head_size=b.head_size,
                   block_size=b.block_size, scale=b.scale, dtype=b.dtype, kv_quant=b.kv_quant,
                   k_scale=b.k_scale, v_scale=b.v_scale)


def cpu_baseline(b, W, target_s: float):
    """Time the oracle on the first k sequences, k sized for ~target_s seconds."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1

    def run(k):
        sb = sub_batch(b, np.arange(k), W)
        t = time.perf_counter()
        oracle.paged_attention(sb.query, sb.key, sb.value, sb.key_cache, sb.value_cache, sb.cum,
                               sb.past, sb.block_table, sb.slot_mapping, num_heads=sb.num_heads,
                               kv_num_heads=sb.kv_num_heads, scale=sb.scale,
                               k_scale=sb.k_scale, v_scale=sb.v_scale)
        return time.perf_counter() - t, W.work(sb)

    t1, _ = run(1)
    k = int(min(b.batch_size, max(1, target_s / max(t1, 1e-3))))
    t, work = run(k)
    reps = 1
    while t < target_s and reps < 1000:  # whole batch is quick: repeat it (t sums the runs)
        dt, _ = run(k)
        t += dt
        reps += 1
    log(f"[bench] cpu oracle: {k} of {b.batch_size} sequences x {reps} in {t:.1f}s "
        f"({threads} BLAS threads)")
    return {"value": round(work["kv_hist_bytes"] * reps / t / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": f"first {k} of {b.batch_size} sequences of {b.name} seed {b.seed}, "
                      f"{reps} run(s) (numpy fp64 oracle incl. its cache copies; {t:.1f} s wall)",
            "seconds": round(t, 2)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="pure_decode")
    ap.add_argument("--also", default="mixed,long_prefill,serving,pure_decode:int8,pure_decode:int4",
                    help="comma list of other workloads to time (empty for none); "
                         "name:int8 or name:int4 times that workload with quantized caches")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--dtype", default="f16", choices=("f16", "bf16"),
                    help="data type of the workloads (the line's dtype field)")
    ap.add_argument("--head-size", type=int, default=0, choices=(0, 64, 128, 256),
                    help="replace the workloads' head size (0: their own)")
    ap.add_argument("--kv-quant", default="none", choices=("none", "int8", "int4"),
                    help="cache element type: the data type, or int8 / int4 codes with "
                         "per-channel scales (history bytes then count one byte / half a byte "
                         "per element)")
    ap.add_argument("--gate", action="store_true",
                    help="pass an output gate: the outputs are multiplied by sigmoid(gate)")
    ap.add_argument("--prologue", type=int, default=0, metavar="ROTARY_DIM",
                    help="fuse the Q/K OffsetRMSNorm and a partial MRoPE over ROTARY_DIM channels "
                         "into the calls (0: none)")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the warm phase (every timed dispatch is then cold, e.g. under a "
                         "profiler whose averages should match the cold figures)")
    ap.add_argument("--scrub", default="read", choices=("read", "rw", "flush"),
                    help="cold protocol cache eviction before each step (see do_scrub)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (for scaling HBM counters)")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                        "COPY_WRITE_CSV"),
                    help="write profiles/traffic_<kernel>_<workload>.json from rocprofv3 "
                         "counter CSVs (with --traffic-kernel, --workload, --copy-calibration)")
    ap.add_argument("--traffic-kernel", default="decode", choices=sorted(KERNEL_SYMBOL))
    args = ap.parse_args()
    VARIANT["suffix"] = variant_suffix(args.dtype, args.head_size, args.kv_quant, args.gate,
                                       args.prologue)
    SCRUB["mode"] = args.scrub

    if args.traffic_from:
        write_traffic(args.traffic_kernel, args.workload, *args.traffic_from,
                      copy_bytes=(args.copy_calibration or 1024) << 20)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library runs on one GPU; the design notes say how it would shard)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_varlen_amd as pa
    import workloads as W

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE per dispatch
        # calibrate the counters used for the kernels' HBM traffic
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "dispatches": args.steps}), flush=True)
        return
    pa.library()  # fail loudly if the HIP library is missing
    scrub = torch.zeros(SCRUB_BYTES // 4, dtype=torch.int32, device="cuda:0")
    variant = dict(dtype=args.dtype, head_size=args.head_size, kv_quant=args.kv_quant,
                   gate=args.gate, warm=not args.no_warm, prologue=args.prologue)

    WORKLOAD_NAME["current"] = args.workload
    b, work, res = time_workload(args.workload, args.steps, args.warmup, args.seed, torch, pa, W,
                                 scrub, **variant)
    head = summarize(args.workload, work, res)
    head_roof = roofline(work, res)
    also = []
    for spec in [x for x in args.also.split(",") if x and x != args.workload]:
        name, _, kvq = spec.partition(":")
        if kvq not in ("", "int8", "int4"):
            raise SystemExit(f"--also {spec}: the cache type after ':' is int8 or int4")
        ov = dict(variant, kv_quant=kvq or args.kv_quant)
        VARIANT["suffix"] = variant_suffix(args.dtype, args.head_size, ov["kv_quant"], args.gate,
                                           args.prologue)
        WORKLOAD_NAME["current"] = name
        ob, owork, ores = time_workload(name, args.steps, args.warmup, args.seed, torch, pa, W,
                                        scrub, **ov)
        entry = summarize(name, owork, ores)
        entry["kv_cache"] = ov["kv_quant"] if ov["kv_quant"] != "none" else args.dtype
        entry["roofline"] = roofline(owork, ores)
        also.append(entry)
        del ob
    VARIANT["suffix"] = variant_suffix(args.dtype, args.head_size, args.kv_quant, args.gate,
                                       args.prologue)

    ms = res["cold"]["median"]
    line = {
        "metric": METRIC,
        "value": round(work["decode_kv_hist_bytes"] / (ms / 1e3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "seed": args.seed, "batch": b.batch_size,
                   "num_tokens": b.num_tokens, "num_heads": b.num_heads,
                   "kv_num_heads": b.kv_num_heads, "head_size": b.head_size,
                   "block_size": b.block_size, "num_blocks": b.num_blocks,
                   "kv_cache": args.dtype if args.kv_quant == "none" else args.kv_quant,
                   "output_gate": bool(args.gate), "qk_prologue_rotary_dim": args.prologue,
                   "kv_hist_bytes": work["kv_hist_bytes"],
                   "protocol": f"cold: 1 GiB scrub ({args.scrub}) before each step, outside "
                               "the events; ms_per_step = median of the per-step event times"},
        "roofline": head_roof,
        "cold": head["cold"],
        "warm": head["warm"],
        "warm_value": None if head["warm"] is None else round(
            work["decode_kv_hist_bytes"] / (head["warm"]["median"] / 1e3) / 1e9, 2),
        "tokens_per_s": head["tokens_per_s"],
        "kernel_us": head["kernel_us"],
        "also": also,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(b, W, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

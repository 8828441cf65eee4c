#!/usr/bin/env python3
"""Benchmark of the FP8-activation x block-scaled FP4 expert GEMM hot path on one MI355X.

A step is one pass of the whole path over one batch: act_quant_fp8 of the token rows, then the
grouped GEMM over the routed rows packed per expert (fp4_grouped_gemm_gather: the packed rows read
their token's codes through row_ids).  The default run measures both halves of the metric in one
process, each on its own workload with its own W warm-up and K timed steps:
  - grouped prefill (8192 tokens, 256 experts, Zipf top-8, k=7168, n=4096): TFLOP/s, timed first;
  - grouped NVFP4 decode step (512 tokens, 256 experts, top-8, k=7168, n=2048): weight-stream TB/s,
    timed right after; this is the line's `value`, and the prefill half is its `prefill` object.
Inputs are resident in HBM before a timed region starts; the weights (2.1 GB and 4.2 GB) exceed the
256 MB Infinity Cache, so every step streams them from HBM.

Prints ONE JSON line on stdout; human-readable detail goes to stderr.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402  (seeded input generators; no torch, no method arithmetic)

METRIC = "FP4 expert GEMM weight-stream TB/s (decode) + TFLOP/s (grouped prefill)"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "fp8": 5000.0}
# The sources of the dominant GEMM kernel of each workload: a recorded traffic figure is used only
# while these files are unchanged since the counters were taken.
GEMM_SOURCES = {
    "config3": ["block_scaled_fp4_quant_amd/csrc/gemm_decode.hip",
                "block_scaled_fp4_quant_amd/csrc/device_common.h"],
    "config4": ["block_scaled_fp4_quant_amd/csrc/gemm_prefill.hip",
                "block_scaled_fp4_quant_amd/csrc/device_common.h"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_text(src: str) -> str:
    """C/C++ source without its comments, whitespace runs collapsed to one space: what the compiler
    sees, so that an edit to comments or layout keeps a recorded measurement valid and any other
    edit does not.  String and character literals are kept as they are."""
    out, i, n = [], 0, len(src)

    def space():
        if out and out[-1] != " ":
            out.append(" ")

    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            space()
            i = n if j < 0 else j + 2
        elif c.isspace():
            space()
            i += 1
        else:
            out.append(c)
            i += 1
    return "".join(out).strip()


def sources_sha(workload: str) -> str:
    """Hash of the code (comments and layout aside) of the kernel sources a traffic record belongs to."""
    h = hashlib.sha256()
    for rel in GEMM_SOURCES[workload]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, layout: str):
    """HBM bytes per GEMM launch measured with rocprofv3 counters for this exact kernel source and
    weight layout, or None when no measurement matches."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload)
    if not ent or ent.get("gemm_sources_sha") != sources_sha(workload) or ent.get("layout", "plain") != layout:
        return None
    return ent.get("hbm_bytes_per_launch")


def algorithmic_bytes(wl) -> dict:
    """Bytes the grouped GEMM must move at minimum: every touched expert's nibble + scale planes
    (+ scale2), the activation codes and scales of the token rows, the routing tables, the f32
    output."""
    T, k = wl.x.shape
    weights = wl.weight_stream_bytes()
    acts = T * k + T * (k // 128) * 4
    tables = wl.R * 4 + (wl.E + 1) * 4 + wl.E * (8 + 8 + 4 + 4)
    out = wl.R * wl.n * 4
    return {"weights": weights, "acts": acts, "tables": tables, "out": out,
            "total": weights + acts + tables + out}


def cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it (model name, family/model/stepping), with the
    number of logical CPUs this process may run on."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" in line:
                    k, v = line.split(":", 1)
                    info.setdefault(k.strip(), v.strip())
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count() or 0
    return (f"{info.get('model name', 'unknown')} (vendor {info.get('vendor_id', '?')}, family "
            f"{info.get('cpu family', '?')}, model {info.get('model', '?')}, stepping {info.get('stepping', '?')}, "
            f"{info.get('cpu MHz', '?')} MHz); {avail} logical CPUs available of {os.cpu_count()}")


def cpu_baseline(wl, budget_s: float, tflops: bool = False):
    """Time the oracle (as it stands) on a bounded sample of the same workload: act-quant of every
    token row, then the grouped GEMM of the first experts' packed rows, adding experts until about
    budget_s of CPU work.  Returns the sample's weight-stream rate in TB/s, or (tflops) its rate in
    TFLOP/s of 2 * rows * k * n, with rows per second in the sample text."""
    import oracle
    oracle.build()
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    codes, scales = oracle.act_quant(wl.x)
    t_aq = time.perf_counter() - t0
    pc, ps = codes[wl.row_ids], scales[wl.row_ids]
    ws = [wl.w_of(e) for e in range(wl.E)]
    ss = [wl.s_of(e) for e in range(wl.E)]
    done_e, rows, t_gemm, nbytes = 0, 0, 0.0, 0
    used_threads = 1
    e = 0
    while e < wl.E and t_gemm + t_aq < budget_s:
        # grow the batch geometrically so that thread start-up is amortised
        e_hi = min(wl.E, e + max(1, done_e))
        r0, r1 = int(wl.offsets[e]), int(wl.offsets[e_hi])
        if tflops and rows > 0 and r1 - r0 > 0:
            # keep the prefill sample near the budget: stop growing once the next batch would overrun
            per_row = t_gemm / rows
            if t_gemm + t_aq + per_row * (r1 - r0) > 1.5 * budget_s:
                e_hi = e + 1
                r1 = int(wl.offsets[e_hi])
        if r1 > r0:
            t1 = time.perf_counter()
            oracle.grouped_gemm(pc, ps, wl.offsets, ws, ss, wl.kinds, wl.scale2, wl.n, row0=r0,
                                row1=r1, threads=threads)
            t_gemm += time.perf_counter() - t1
            used_threads = max(used_threads, min(threads, r1 - r0))
        for ee in range(e, e_hi):
            if wl.offsets[ee + 1] > wl.offsets[ee]:
                nbytes += wl.n * wl.k // 2 + wl.n * wl.k // workloads.GROUP_SIZE[int(wl.kinds[ee])] + 4
        rows += r1 - r0
        done_e = e_hi
        e = e_hi
    frac = rows / wl.R
    elapsed = t_gemm + t_aq * frac
    sample = (f"oracle act-quant of all {wl.x.shape[0]} token rows (time pro-rated to the sampled share of "
              f"packed rows) + f64 grouped GEMM of experts 0..{done_e - 1} ({rows} of {wl.R} packed rows, "
              f"{nbytes} weight bytes) of the same workload; {t_gemm:.1f} s GEMM + {t_aq:.1f} s act-quant; "
              f"{rows / elapsed:.1f} rows/s")
    if tflops:
        value, unit = 2.0 * rows * wl.k * wl.n / elapsed / 1e12, "TFLOP/s"
    else:
        value, unit = nbytes / elapsed / 1e12, "TB/s"
    return {"value": value, "unit": unit, "cores": used_threads, "kind": "oracle", "cpu": cpu_model(),
            "rows_per_s": round(rows / elapsed, 2), "sample": sample}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="both",
                    choices=["both", "config3", "config4", "chain4", "w4a4", "config1", "config2", "peaks", "floors"],
                    help="both (default): the grouped prefill GEMM step, then the grouped decode GEMM step, "
                         "reported in one line (decode = value, prefill = the `prefill` object); "
                         "config3: grouped decode GEMM alone; config4: grouped prefill GEMM alone; chain4: the "
                         "whole prefill expert layer from router logits (top-k, packing, gate/up GEMM, "
                         "swiglu+quant, down GEMM, combine); w4a4: the W4A4 variant on one NVFP4 "
                         "expert of the prefill shape, beside the FP8 path on the same inputs")
    ap.add_argument("--gate-up", default="fused", choices=["fused", "unfused"],
                    help="chain4 only: the gate/up GEMM with the activation and its quantization in "
                         "its epilogue (fused), or the GEMM writing f32 gate/up values followed by "
                         "swiglu_quant_fp8 (unfused)")
    ap.add_argument("--tokens", type=int, default=0,
                    help="config3 only: a decode step of the first T tokens (top-8 over the same 256 "
                         "experts; default all 512)")
    ap.add_argument("--rows", type=int, default=8,
                    help="config1 only: activation rows g (1, 2, 4 or 8)")
    ap.add_argument("--cached", action="store_true",
                    help="config1/config2: one copy of the weights (served from the Infinity Cache "
                         "after the first step) instead of rotating over >= 560 MB of copies")
    ap.add_argument("--layout", default="swizzled", choices=["swizzled", "plain"],
                    help="config3/config4/chain4: expert planes in the swizzled layout (fp4_weight_swizzle, "
                         "run once at load time before the timed region) or as the plain [n, k/2] and "
                         "[n, k/gs] planes")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the cpu_baseline leg (0 disables it)")
    ap.add_argument("--per-step", action="store_true",
                    help="grouped workloads: list every timed step's GEMM time (HIP events) on stderr")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="after timing, run 3 plain device copies of MIB MiB (a known-size kernel "
                         "for scaling the HBM byte counters of a profiler run)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_scaled_fp4_quant_amd as fp4

    if not torch.cuda.is_available():
        print("bench.py needs a HIP GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log(f"library: {fp4.version()}  device: {torch.cuda.get_device_name(dev)}")

    if args.workload == "chain4":
        return run_chain(args, torch, fp4, dev)
    if args.workload == "w4a4":
        return run_w4a4(args, torch, fp4, dev)
    if args.workload in ("config1", "config2"):
        return run_single_expert(args, torch, fp4, dev)
    if args.workload == "floors":
        return run_floors(args, torch, dev)
    if args.workload == "peaks":
        return run_peaks(args, torch, dev)

    return run_grouped(args, torch, fp4, dev)


def input_hashes(wl) -> dict:
    """sha256 of every generated input array of a grouped workload (as generated, before upload)."""
    arrs = {"x": wl.x, "row_ids": wl.row_ids, "offsets": wl.offsets, "kinds": wl.kinds,
            "scale2": wl.scale2, "w_bank": wl.w_bank, "s_bank": wl.s_bank}
    if wl.logits is not None:
        arrs["logits"] = wl.logits
    return {k: hashlib.sha256(np.ascontiguousarray(v).data).hexdigest() for k, v in arrs.items()}


def make_grouped(name: str, tokens: int):
    if name == "config4":
        return workloads.config4()
    wl = workloads.config3()
    if 0 < tokens < wl.x.shape[0]:
        rid, off = workloads.route_topk(wl.logits[:tokens], 8)
        wl = dataclasses.replace(wl, x=np.ascontiguousarray(wl.x[:tokens]), row_ids=rid, offsets=off,
                                 logits=wl.logits[:tokens],
                                 name=f"config3 experts, decode step of {tokens} tokens: E=256, top-8, k=7168, n=2048")
    return wl


class GroupedRun:
    """A grouped workload resident on the device (planes swizzled at load time unless --layout
    plain), with the buffers of one step."""

    def __init__(self, wl, layout, torch, fp4, dev):
        self.wl = wl
        self.fp4 = fp4
        self.x = torch.from_numpy(wl.x).to(dev)
        self.row_ids = torch.from_numpy(wl.row_ids).to(dev)
        self.offsets = torch.from_numpy(wl.offsets).to(dev)
        self.kinds = torch.from_numpy(wl.kinds).to(dev)
        self.scale2 = torch.from_numpy(wl.scale2.astype(np.float32)).to(dev)
        w_bank = torch.from_numpy(wl.w_bank).to(dev)
        s_bank = torch.from_numpy(wl.s_bank).to(dev)
        self.w_ptrs = torch.from_numpy((w_bank.data_ptr() + wl.w_off).astype(np.int64)).to(dev)
        self.s_ptrs = torch.from_numpy((s_bank.data_ptr() + wl.s_off).astype(np.int64)).to(dev)
        if layout == "swizzled":
            w_bank, s_bank, self.w_ptrs, self.s_ptrs, self.kinds = swizzle_bank(wl, torch, fp4, dev, w_bank, s_bank)
        self.banks = (w_bank, s_bank)
        T, k = wl.x.shape
        self.codes = torch.empty((T, k), dtype=torch.uint8, device=dev)
        self.scales = torch.empty((T, k // 128), dtype=torch.float32, device=dev)
        self.out = torch.empty((wl.R, wl.n), dtype=torch.float32, device=dev)

    def act_quant(self, stream):
        self.fp4.act_quant_fp8(self.x, self.codes, self.scales, stream=stream)

    def gemm(self, stream):
        self.fp4.fp4_grouped_gemm_gather(self.codes, self.scales, self.row_ids, self.offsets, self.w_ptrs, self.s_ptrs,
                                         self.kinds, self.scale2, self.wl.n, out=self.out, stream=stream)

    def time(self, torch, warmup: int, steps: int) -> dict:
        """W untimed steps, then K timed ones with HIP events on the launch stream before the
        act-quant, between the two launches and after the GEMM."""
        stream = torch.cuda.current_stream()
        for _ in range(warmup):
            self.act_quant(stream)
            self.gemm(stream)
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        for i in range(steps):
            ev[i][0].record(stream)
            self.act_quant(stream)
            ev[i][1].record(stream)
            self.gemm(stream)
            ev[i][2].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        gemm_all = np.array([e[1].elapsed_time(e[2]) for e in ev])
        return {"step_ms": ev[0][0].elapsed_time(ev[steps - 1][2]) / steps, "wall_ms": wall * 1e3 / steps,
                "gemm_us_each": [round(float(v) * 1e3, 1) for v in gemm_all],
                "aq_ms": float(np.mean([e[0].elapsed_time(e[1]) for e in ev])),
                "gemm_ms": float(np.mean(gemm_all)), "gemm_ms_min": float(np.min(gemm_all)),
                "gemm_pct": {f"p{q}": round(float(np.percentile(gemm_all, q)) * 1e3, 2) for q in (10, 50, 90)}}


def half_result(name, wl, m, args, hashes) -> dict:
    """The JSON fields of one half: the decode half is HBM-bound (weight-stream TB/s), the prefill
    half matrix-core-bound (TFLOP/s against the bf16/f16 class issued and against the FP8 peak)."""
    alg = algorithmic_bytes(wl)
    flops = 2.0 * wl.R * wl.k * wl.n
    ws_bytes = alg["weights"]
    gemm_s = m["gemm_ms"] * 1e-3
    traffic = None if args.tokens and name == "config3" else recorded_traffic(name, args.layout)
    T = wl.x.shape[0]
    config = {"workload": wl.name, "tokens": int(T), "experts": int(wl.E), "top_k": 8,
              "routed_rows": int(wl.R), "k": int(wl.k), "n": int(wl.n), "weight_layout": args.layout,
              "weight_stream_bytes": int(ws_bytes), "algorithmic_bytes": int(alg["total"]), "flops": flops,
              "gemm_us": round(m["gemm_ms"] * 1e3, 2), "gemm_us_min": round(m["gemm_ms_min"] * 1e3, 2),
              "gemm_us_percentiles": m["gemm_pct"], "act_quant_us": round(m["aq_ms"] * 1e3, 2),
              "inputs_sha256": hashes}
    if name == "config3":
        achieved = alg["total"] / gemm_s / 1e9
        log(f"[decode] timed {args.steps} steps: {m['step_ms']:.4f} ms/step (act_quant {m['aq_ms'] * 1e3:.1f} us, "
            f"GEMM {m['gemm_ms'] * 1e3:.1f} us avg / {m['gemm_ms_min'] * 1e3:.1f} us min); weight stream "
            f"{ws_bytes / gemm_s / 1e12:.3f} TB/s in the GEMM; algorithmic bytes {alg['total'] / 1e9:.3f} GB -> "
            f"{achieved:.0f} GB/s ({achieved / HBM_PEAK_GBS:.1%} of 8 TB/s)")
        return {"value": round(ws_bytes / (m["step_ms"] * 1e-3) / 1e12, 4), "unit": "TB/s",
                "ms_per_step": round(m["step_ms"], 4), "config": config,
                "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}}
    tf = flops / gemm_s / 1e12
    log(f"[prefill] timed {args.steps} steps: {m['step_ms']:.4f} ms/step (act_quant {m['aq_ms'] * 1e3:.1f} us, "
        f"GEMM {m['gemm_ms'] * 1e3:.1f} us avg / {m['gemm_ms_min'] * 1e3:.1f} us min); {tf:.1f} TFLOP/s = "
        f"{tf / MFMA_PEAK_TFLOPS['f16']:.1%} of the 2.5 PFLOP/s bf16/f16 class, "
        f"{tf / MFMA_PEAK_TFLOPS['fp8']:.1%} of the 5.0 PFLOP/s FP8 figure")
    return {"value": round(flops / (m["step_ms"] * 1e-3) / 1e12, 4), "unit": "TFLOP/s",
            "ms_per_step": round(m["step_ms"], 4), "config": config,
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_PEAK_TFLOPS["f16"],
                         "unit": "TFLOP/s", "frac": round(tf / MFMA_PEAK_TFLOPS["f16"], 4), "traffic": traffic,
                         "peak_is": "dense bf16/f16 MFMA, the class the kernel issues"},
            "roofline_fp8": {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_PEAK_TFLOPS["fp8"],
                             "unit": "TFLOP/s", "frac": round(tf / MFMA_PEAK_TFLOPS["fp8"], 4),
                             "peak_is": "dense FP8 (F8F6F4) MFMA, the method's own roofline"}}


def run_grouped(args, torch, fp4, dev):
    """The grouped workloads: `both` (the default: the prefill half, then the decode half, in one
    line), `config3` or `config4` alone."""
    halves = ["config4", "config3"] if args.workload == "both" else [args.workload]
    runs, wls, hashes = {}, {}, {}
    for name in halves:
        t0 = time.perf_counter()
        wl = make_grouped(name, args.tokens)
        hashes[name] = input_hashes(wl)
        runs[name] = GroupedRun(wl, args.layout, torch, fp4, dev)
        wls[name] = wl
        torch.cuda.synchronize()
        log(f"workload: {wl.name}  (generated, hashed and uploaded in {time.perf_counter() - t0:.1f} s)")
    meas = {}
    for name in halves:
        # The decode half is timed right after the prefill half.  From an idle GPU the first ~40 ms
        # of any load run at a lower core clock (the decode GEMM then takes up to 470 us instead of
        # 345 us in dispatches 5-25); after the prefill half's steps the decode half's W warm-up
        # steps start at the settled clock.  `--workload config3` times the decode half alone.
        meas[name] = runs[name].time(torch, args.warmup, args.steps)
        if args.per_step:
            each = meas[name]["gemm_us_each"]
            log(f"[{name}] GEMM us of each timed step:")
            for i in range(0, len(each), 10):
                log(f"  {i:4d}: " + " ".join(f"{v:7.1f}" for v in each[i:i + 10]))
    res = {name: half_result(name, wls[name], meas[name], args, hashes[name]) for name in halves}
    head = "config3" if "config3" in res else "config4"
    h = res[head]
    result = {
        "metric": METRIC, "value": h["value"], "unit": h["unit"], "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": h["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8xfp4->f32", "data": "synthetic",
        "config": h["config"], "roofline": h["roofline"], "cpu_baseline": None,
    }
    if head == "config4":
        result["roofline_fp8"] = h["roofline_fp8"]
    if len(halves) == 2:
        p = res["config4"]
        result["config"]["timed_after"] = "the prefill half (its W warm-up and K timed steps) in the same process"
        result["prefill"] = {"metric": "grouped prefill TFLOP/s", "value": p["value"], "unit": "TFLOP/s",
                             "ms_per_step": p["ms_per_step"], "steps": args.steps, "warmup": args.warmup,
                             "config": p["config"], "roofline": p["roofline"], "roofline_fp8": p["roofline_fp8"],
                             "cpu_baseline": None}
    if "config4" in halves:
        # Context for the prefill fraction: the matrix cores' sustained rate on this GPU in this run
        # (after the timed halves, so it cannot affect them).  Full matrix-core load is power-limited,
        # so this is well below the published 2.5 PFLOP/s that `roofline` keeps as its peak.
        target = result["prefill"] if len(halves) == 2 else result
        try:
            loop = mfma_loop_rates(torch, dev, lambda fn, reps: event_timed(torch, fn, reps),
                                   which=("changing_operands",))["changing_operands"]
            ach = res["config4"]["roofline"]["achieved"]
            target["roofline_sustained"] = {
                "bound": "mfma", "achieved": ach, "peak": loop["tflops"], "unit": "TFLOP/s",
                "frac": round(ach / loop["tflops"], 4), "clock_mhz": loop["clock_mhz"],
                "peak_is": "register-only f16 32x32x16 MFMA loop on this GPU in the same run (operands "
                           "changing every round, 2 wavefronts per SIMD), at the clock it measures"}
        except (OSError, SystemExit, RuntimeError) as exc:
            log(f"sustained MFMA rate not measured: {exc}")
            target["roofline_sustained"] = None
    if args.calibrate_copy > 0:
        nbytes = args.calibrate_copy << 20
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)          # an elementwise kernel: reads and writes nbytes
        torch.cuda.synchronize()
        log(f"calibration: 3 copies of {nbytes} bytes (read {nbytes}, write {nbytes} each)")
    del runs
    if args.cpu_budget > 0:
        for name in halves:
            log(f"cpu_baseline [{name}]: timing the oracle for about {args.cpu_budget:.0f} s ...")
            cb = cpu_baseline(wls[name], args.cpu_budget, tflops=(name == "config4"))
            log(f"cpu_baseline [{name}]: {cb}")
            if name == head:
                result["cpu_baseline"] = cb
            else:
                result["prefill"]["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


def swizzle_bank(wl, torch, fp4, dev, w_bank, s_bank):
    """Every expert's planes rewritten by fp4_weight_swizzle into new banks (load-time work, before
    any timing); returns the banks, their address tables and the kinds with the layout flag."""
    sizes = [fp4.swizzled_plane_bytes(int(kd), wl.n, wl.k) for kd in wl.kinds]
    w_off = np.concatenate([[0], np.cumsum([a for a, _ in sizes])]).astype(np.int64)
    s_off = np.concatenate([[0], np.cumsum([(b + 255) // 256 * 256 for _, b in sizes])]).astype(np.int64)
    w_swz = torch.empty(int(w_off[-1]), dtype=torch.uint8, device=dev)
    s_swz = torch.empty(int(s_off[-1]), dtype=torch.uint8, device=dev)
    gs = {workloads.NVFP4: 16, workloads.MXFP4: 32}
    for e, kd in enumerate(wl.kinds):
        kd = int(kd)
        wp = w_bank[int(wl.w_off[e]):int(wl.w_off[e]) + wl.n * wl.k // 2].view(wl.n, wl.k // 2)
        sp = s_bank[int(wl.s_off[e]):int(wl.s_off[e]) + wl.n * wl.k // gs[kd]].view(wl.n, wl.k // gs[kd])
        fp4.fp4_weight_swizzle(wp, sp, kd, w_out=w_swz[int(w_off[e]):int(w_off[e + 1])],
                               s_out=s_swz[int(s_off[e]):int(s_off[e]) + sizes[e][1]])
    torch.cuda.synchronize()
    w_ptrs = torch.from_numpy((w_swz.data_ptr() + w_off[:-1]).astype(np.int64)).to(dev)
    s_ptrs = torch.from_numpy((s_swz.data_ptr() + s_off[:-1]).astype(np.int64)).to(dev)
    kinds = torch.from_numpy((wl.kinds | fp4.SWIZZLED).astype(np.int32)).to(dev)
    return w_swz, s_swz, w_ptrs, s_ptrs, kinds


def run_single_expert(args, torch, fp4, dev):
    """One expert of a decode shape (config1: MXFP4, g rows, k=7168, n=2048; config2: NVFP4, 16 rows,
    k=2048, n=7168): act_quant_fp8 + fp4_expert_gemm per step.  A single expert's 8 MB fits the
    256 MB Infinity Cache, so the steps rotate over enough copies of the planes (>= 72 and
    >= 560 MB) that every step streams its weights from HBM.  value = weight-stream TB/s."""
    wl = workloads.config1(args.rows) if args.workload == "config1" else workloads.config2()
    ex = wl.expert
    g, k = wl.x.shape
    n = ex.w.shape[0]
    log(f"workload: {wl.name}")
    x = torch.from_numpy(wl.x).to(dev)
    w0, s0 = torch.from_numpy(ex.w).to(dev), torch.from_numpy(ex.s).to(dev)
    wbytes = ex.w.size + ex.s.size + (4 if ex.kind == workloads.NVFP4 else 0)
    ncopy = 1 if args.cached else max(72, -(-(560 << 20) // wbytes))
    if args.layout == "swizzled":
        planes = [fp4.fp4_weight_swizzle(w0, s0, ex.kind) for _ in range(ncopy)]
        kind = ex.kind | fp4.SWIZZLED
    else:
        planes = [(w0.clone(), s0.clone()) for _ in range(ncopy)]
        kind = ex.kind
    codes = torch.empty((g, k), dtype=torch.uint8, device=dev)
    scales = torch.empty((g, k // 128), dtype=torch.float32, device=dev)
    out = torch.empty((g, n), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        if ev:
            ev[0].record(stream)
        fp4.act_quant_fp8(x, codes, scales, stream=stream)
        if ev:
            ev[1].record(stream)
        w, sc = planes[i % ncopy]
        fp4.fp4_expert_gemm(codes, scales, w, sc, ex.scale2, kind, out=out, stream=stream, n=n)
        if ev:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for i in range(K):
        step(args.warmup + i, ev[i])
    torch.cuda.synchronize()
    step_ms = ev[0][0].elapsed_time(ev[K - 1][2]) / K
    aq_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    gemm_all = np.array([e[1].elapsed_time(e[2]) for e in ev])
    gemm_ms = float(np.mean(gemm_all))
    gemm_pct = {f"p{q}": round(float(np.percentile(gemm_all, q)) * 1e3, 2) for q in (10, 50, 90)}
    alg = wbytes + g * k + g * (k // 128) * 4 + g * n * 4
    achieved = alg / (gemm_ms * 1e-3) / 1e9
    log(f"{K} steps: {step_ms * 1e3:.2f} us/step (act_quant {aq_ms * 1e3:.2f} us, GEMM {gemm_ms * 1e3:.2f} us); "
        f"{ncopy} weight copies rotated")
    import oracle
    oracle.build()
    # the oracle splits an expert's rows over its threads: one thread per row, up to the host's count
    threads = max(1, min(oracle.default_threads(), int(g)))
    t0 = time.perf_counter()
    rc, rs = oracle.act_quant(wl.x)
    oracle.expert_gemm(rc, rs, ex.w, ex.s, ex.scale2, ex.kind, threads=threads)
    t_cpu = time.perf_counter() - t0
    result = {
        "metric": METRIC, "value": round(wbytes / (step_ms * 1e-3) / 1e12, 4), "unit": "TB/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(step_ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8xfp4->f32", "data": "synthetic",
        "config": {"workload": wl.name, "rows": int(g), "k": int(k), "n": int(n), "weight_layout": args.layout,
                   "weight_copies_rotated": int(ncopy), "cached": bool(args.cached),
                   "weight_stream_bytes": int(wbytes), "gemm_us": round(gemm_ms * 1e3, 2),
                   "gemm_us_percentiles": gemm_pct, "act_quant_us": round(aq_ms * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": {"value": wbytes / t_cpu / 1e12, "unit": "TB/s", "cores": threads, "kind": "oracle",
                         "cpu": cpu_model(),
                         "sample": f"oracle act-quant + f64 expert GEMM of the whole step, {threads} threads "
                                   f"(one per row), {t_cpu:.2f} s"},
    }
    print(json.dumps(result), flush=True)


def run_floors(args, torch, dev):
    """Practical floors of a single-expert launch: an almost empty launch (torch.cuda._sleep(0)), a
    streaming read of one expert's plane bytes by the library's own memory-bound kernel (act_quant_fp8
    over an f32 input of that size: one 16-byte load per lane, 1 byte written per 4 read), and a
    device copy of the same bytes (torch copy_).  Config1 planes: 7,798,784 B; config2: 8,257,540 B
    (8,257,536 B of f32 rows here).  Inputs rotate over >= 72 copies (>= 560 MB, more than the
    Infinity Cache) so that every launch streams from HBM.  HIP events per launch; the kernel
    durations come from a kernel trace of the same command."""
    import block_scaled_fp4_quant_amd as fp4
    K = max(args.steps, 200)
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        for i in range(20):
            fn(i)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for i in range(reps):
            fn(i)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        d = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]) * 1e3
        return float(np.mean(d)), float(np.median(d))

    res = {}
    res["empty_launch_us"] = timed(lambda i: torch.cuda._sleep(0), K)
    for name, rows in (("config1", 15232), ("config2", 16128)):
        nbytes = rows * 128 * 4
        ncopy = max(72, -(-(560 << 20) // nbytes))
        bufs = [torch.ones((rows, 128), dtype=torch.float32, device=dev) for _ in range(ncopy)]
        codes = torch.empty((rows, 128), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, 1), dtype=torch.float32, device=dev)
        dsts = [torch.empty((rows, 128), dtype=torch.float32, device=dev) for _ in range(8)]
        res[f"{name}_read_us"] = timed(lambda i: fp4.act_quant_fp8(bufs[i % ncopy], codes, scales, stream=stream), K)
        res[f"{name}_copy_us"] = timed(lambda i: dsts[i % 8].copy_(bufs[i % ncopy]), K)
        del bufs, dsts
    for k_, (mean, p50) in res.items():
        log(f"{k_}: mean {mean:.2f} us, p50 {p50:.2f} us (events)")
    result = {
        "metric": "single-expert launch floors (empty launch, plane-sized streaming read and copy)",
        "value": round(res["config1_read_us"][1], 3), "unit": "us", "n_gpus": 1, "steps": K, "warmup": 20,
        "ms_per_step": round(res["config1_read_us"][1] / 1e3, 6), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "floors: torch.cuda._sleep(0); act_quant_fp8 and copy_ over one expert's plane "
                               "bytes of f32, rotated over >= 560 MB",
                   **{k_: {"mean": round(v[0], 2), "p50": round(v[1], 2)} for k_, v in res.items()}},
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


def event_timed(torch, fn, reps):
    """Average seconds per call of fn over reps calls (HIP events on the current stream), after a
    few untimed calls."""
    for _ in range(max(3, reps // 4)):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


def mfma_loop_rates(torch, dev, timed, which=("changing_operands", "constant_operands")):
    """Sustained dense f16 MFMA rate and core clock from the register-only loop in
    libfp4moe_probe.so (two workgroups of four wavefronts per compute unit, 32x32x16 MFMAs), with
    operands that change every round and/or with constant operands.  The clock is each workgroup's
    s_memtime cycles over its s_memrealtime (100 MHz) ticks; reported as the median over workgroups."""
    import ctypes
    path = os.path.join(ROOT, "block_scaled_fp4_quant_amd", "libfp4moe_probe.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is missing: build it with python -m block_scaled_fp4_quant_amd.build")
    L = ctypes.CDLL(path)
    fn = L.fp4moe_probe_mfma_loop
    fn.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    nblocks, iters = 2 * cus, 20000
    sink = torch.empty(nblocks * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(nblocks * 4, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    flops = nblocks * 4 * iters * 4 * 2 * 32 * 32 * 16
    out = {"workgroups": nblocks, "waves_per_simd": 2, "iters": iters}
    for name, toggle in (("changing_operands", 1), ("constant_operands", 0)):
        if name not in which:
            continue

        def launch():
            rc = fn(iters, toggle, nblocks, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(clocks.data_ptr()),
                    ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"fp4moe_probe_mfma_loop returned {rc}")
        timed(launch, 20)                                 # about 60 ms of load before the timed launches
        t = timed(launch, 20)
        c = clocks.cpu().numpy().view(np.uint64).reshape(nblocks, 4).astype(np.float64)
        mhz = float(np.median((c[:, 1] - c[:, 0]) / (c[:, 3] - c[:, 2]) * 100.0))
        tf = flops / t / 1e12
        out[name] = {"tflops": round(tf, 1), "clock_mhz": round(mhz, 0),
                     "flops_per_clock_per_cu": round(tf * 1e12 / (mhz * 1e6) / cus, 1)}
        log(f"f16 MFMA loop, {name.replace('_', ' ')}: {tf:.0f} TFLOP/s at {mhz:.0f} MHz")
    return out


def run_peaks(args, torch, dev):
    """The roofline denominators re-measured on this GPU: a device-to-device copy of 4 GiB (HBM read
    + write), a read-only reduction of 4 GiB and a dense bf16 matrix product 8192^3 (hipBLASLt), all
    torch kernels, and the register-only f16 MFMA loop of libfp4moe_probe.so.  Not part of the method: context for the fractions of
    the published figures (8 TB/s, 2.5 PFLOP/s) that the other workloads report."""
    nbytes = 4 << 30
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).uniform_()
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, dtype=torch.bfloat16, device=dev)
    b = torch.randn(8192, 8192, dtype=torch.bfloat16, device=dev)

    def timed(fn, reps):
        return event_timed(torch, fn, reps)

    t_copy = timed(lambda: dst.copy_(src), 20)
    t_read = timed(lambda: src.sum(), 20)
    t_mm = timed(lambda: torch.mm(a, b), 50)
    copy_gbs = 2 * nbytes / t_copy / 1e9
    read_gbs = nbytes / t_read / 1e9
    mm_tf = 2 * 8192 ** 3 / t_mm / 1e12
    log(f"copy {copy_gbs:.0f} GB/s (read+write), read {read_gbs:.0f} GB/s, bf16 mm {mm_tf:.0f} TFLOP/s")
    del src, dst
    mfma = mfma_loop_rates(torch, dev, timed)
    result = {
        "metric": "roofline denominators re-measured (copy GB/s, read GB/s, bf16 GEMM TFLOP/s, f16 MFMA loop)",
        "value": round(read_gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": 20, "warmup": 5,
        "ms_per_step": round(t_read * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32 / bf16", "data": "synthetic",
        "config": {"workload": "peaks: 4 GiB f32 copy and sum, bf16 mm 8192^3",
                   "copy_gbs": round(copy_gbs, 1), "read_gbs": round(read_gbs, 1),
                   "bf16_mm_tflops": round(mm_tf, 1), "f16_mfma_loop": mfma, "published_hbm_gbs": HBM_PEAK_GBS,
                   "published_bf16_tflops": MFMA_PEAK_TFLOPS["f16"]},
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


def upload_bank(gw, torch, dev):
    w_bank = torch.from_numpy(gw.w_bank).to(dev)
    s_bank = torch.from_numpy(gw.s_bank).to(dev)
    w_ptrs = torch.from_numpy((w_bank.data_ptr() + gw.w_off).astype(np.int64)).to(dev)
    s_ptrs = torch.from_numpy((s_bank.data_ptr() + gw.s_off).astype(np.int64)).to(dev)
    return w_bank, s_bank, w_ptrs, s_ptrs, torch.from_numpy(gw.scale2.astype(np.float32)).to(dev)


def run_chain(args, torch, fp4, dev):
    """The whole prefill expert layer from router logits to the combined output: route_softmax_topk
    -> route_pack -> act_quant -> gate/up grouped GEMM -> swiglu_quant (x routing weight) -> down
    grouped GEMM -> moe_combine.  value = TFLOP/s of the two GEMMs over the whole step; the roofline
    is the dominant kernel's (the gate/up GEMM); every other launch's time is reported beside it."""
    t0 = time.perf_counter()
    ch = workloads.config4_chain()
    log(f"workload: {ch.name}  (generated in {time.perf_counter() - t0:.1f} s)")
    E, top = len(ch.kinds), 8
    logits = torch.from_numpy(ch.logits).to(dev)
    x = torch.from_numpy(ch.x).to(dev)
    kinds = torch.from_numpy(ch.kinds).to(dev)
    up = upload_bank(ch.up, torch, dev)
    dn = upload_bank(ch.down, torch, dev)
    if args.layout == "swizzled":
        ub, us, uw, usp, kinds = swizzle_bank(ch.up, torch, fp4, dev, up[0], up[1])
        up = (ub, us, uw, usp, up[4])
        db, ds, dw, dsp, _ = swizzle_bank(ch.down, torch, fp4, dev, dn[0], dn[1])
        dn = (db, ds, dw, dsp, dn[4])
    T, Hd = ch.x.shape
    R, I = T * top, ch.inter
    ids = torch.empty((T, top), dtype=torch.int32, device=dev)
    tw = torch.empty((T, top), dtype=torch.float32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_ids = torch.empty(R, dtype=torch.int32, device=dev)
    pair_rows = torch.empty((T, top), dtype=torch.int32, device=dev)
    rw = torch.empty(R, dtype=torch.float32, device=dev)
    ws = torch.empty(fp4.route_pack_workspace_size(T, E), dtype=torch.uint8, device=dev)
    codes = torch.empty((T, Hd), dtype=torch.uint8, device=dev)
    scales = torch.empty((T, Hd // 128), dtype=torch.float32, device=dev)
    gu = torch.empty((R, 2 * I), dtype=torch.float32, device=dev)
    hc = torch.empty((R, I), dtype=torch.uint8, device=dev)
    hs = torch.empty((R, I // 128), dtype=torch.float32, device=dev)
    y = torch.empty((R, Hd), dtype=torch.float32, device=dev)
    out = torch.empty((T, Hd), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    fused = args.gate_up == "fused"
    if fused:
        names = ["route_topk", "route_pack", "act_quant", "gate/up GEMM+swiglu+quant", "down GEMM", "combine"]
    else:
        names = ["route_topk", "route_pack", "act_quant", "gate/up GEMM", "swiglu+quant", "down GEMM", "combine"]

    def launches():
        yield lambda: fp4.route_softmax_topk(logits, top, ids=ids, weights=tw, stream=stream)
        yield lambda: fp4.route_pack(ids, E, tw, offsets, row_ids, pair_rows, rw, ws, stream=stream)
        yield lambda: fp4.act_quant_fp8(x, codes, scales, stream=stream)
        if fused:
            yield lambda: fp4.fp4_grouped_gemm_swiglu_quant(codes, scales, row_ids, offsets, up[2], up[3], kinds,
                                                            up[4], I, ch.limit, row_weights=rw, h_codes=hc,
                                                            h_scales=hs, stream=stream)
        else:
            yield lambda: fp4.fp4_grouped_gemm_gather(codes, scales, row_ids, offsets, up[2], up[3], kinds, up[4],
                                               2 * I, out=gu, stream=stream)
            yield lambda: fp4.swiglu_quant_fp8(gu, ch.limit, row_weights=rw, codes=hc, scales=hs, stream=stream)
        yield lambda: fp4.fp4_grouped_gemm_gather(hc, hs, None, offsets, dn[2], dn[3], kinds, dn[4], Hd, out=y,
                                           stream=stream)
        yield lambda: fp4.moe_combine(y, pair_rows, out=out, stream=stream)

    for _ in range(args.warmup):
        for f in launches():
            f()
    torch.cuda.synchronize()
    if not (torch.equal(offsets.cpu(), torch.from_numpy(ch.offsets))
            and torch.equal(row_ids.cpu(), torch.from_numpy(ch.row_ids))):
        raise SystemExit("device routing tables differ from the workload's")
    K, L = args.steps, len(names)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(L + 1)] for _ in range(K)]
    wall0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        for j, f in enumerate(launches()):
            f()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = ev[0][0].elapsed_time(ev[K - 1][L]) / K
    part = [float(np.mean([e[j].elapsed_time(e[j + 1]) for e in ev])) for j in range(L)]
    us = dict(zip(names, part))
    f_up, f_dn = 2.0 * R * Hd * 2 * I, 2.0 * R * I * Hd
    sw_bytes = R * I * (8 + 1) + R * (I // 128) * 4 + R * 4
    cb_bytes = R * Hd * 4 + T * Hd * 4 + T * top * 4
    log(f"timed {K} steps: wall {wall * 1e3 / K:.3f} ms/step, events {step_ms:.3f} ms/step")
    log("  " + ", ".join(f"{n} {p * 1e3:.1f} us" for n, p in zip(names, part)))
    t_up = us["gate/up GEMM+swiglu+quant" if fused else "gate/up GEMM"]
    tf_up = f_up / (t_up * 1e-3) / 1e12
    sw_gbs = None if fused else sw_bytes / (us["swiglu+quant"] * 1e-3) / 1e9
    cb_gbs = cb_bytes / (us["combine"] * 1e-3) / 1e9
    log(f"gate/up{' (fused with swiglu+quant)' if fused else ''} {tf_up:.1f} TFLOP/s, down "
        f"{f_dn / (us['down GEMM'] * 1e-3) / 1e12:.1f} TFLOP/s, "
        + ("" if fused else f"swiglu+quant {sw_gbs:.0f} GB/s ({sw_gbs / HBM_PEAK_GBS:.1%} of 8 TB/s), ")
        + f"combine {cb_gbs:.0f} GB/s ({cb_gbs / HBM_PEAK_GBS:.1%})")
    value = (f_up + f_dn) / (step_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC, "value": round(value, 4), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8xfp4->f32", "data": "synthetic",
        "config": {"workload": ch.name, "tokens": int(T), "experts": int(E), "top_k": top,
                   "routed_rows": int(R), "hidden": int(Hd), "inter": int(I),
                   "gate_up": args.gate_up, "weight_layout": args.layout, "us": {n: round(p * 1e3, 2) for n, p in zip(names, part)},
                   "swiglu_quant_gbs": None if fused else round(sw_gbs, 1), "combine_gbs": round(cb_gbs, 1)},
        "roofline": {"bound": "mfma", "achieved": round(tf_up, 1), "peak": MFMA_PEAK_TFLOPS["f16"],
                     "unit": "TFLOP/s", "frac": round(tf_up / MFMA_PEAK_TFLOPS["f16"], 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


def run_w4a4(args, torch, fp4, dev):
    """The W4A4 variant: act_quant_fp4 (two-level) + w4a4_gemm on one NVFP4 expert of the prefill
    gate/up shape (n = 4096, k = 7168) over 8192 tokens of 0.1 U[0, 1) activations, timed beside
    act_quant_fp8 + fp4_expert_gemm on the same activations and weights."""
    T, n, k = 8192, 4096, 7168
    x_np, ex = workloads.w4a4_case(7, T, n, k, "uniform")
    x = torch.from_numpy(x_np).to(dev)
    w = torch.from_numpy(ex.w).to(dev)
    sc = torch.from_numpy(ex.s).to(dev)
    codes4 = torch.empty((T, k // 2), dtype=torch.uint8, device=dev)
    micro = torch.empty((T, k // 16), dtype=torch.uint8, device=dev)
    rs = torch.empty(T, dtype=torch.float32, device=dev)
    codes8 = torch.empty((T, k), dtype=torch.uint8, device=dev)
    scales8 = torch.empty((T, k // 128), dtype=torch.float32, device=dev)
    out = torch.empty((T, n), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    legs = {
        "act_quant_fp4": lambda: fp4.act_quant_fp4(x, True, None, codes4, micro, rs, stream=stream),
        "w4a4_gemm": lambda: fp4.w4a4_gemm(codes4, micro, rs, w, sc, ex.scale2, out=out, stream=stream),
        "act_quant_fp8": lambda: fp4.act_quant_fp8(x, codes8, scales8, stream=stream),
        "fp4_expert_gemm": lambda: fp4.fp4_expert_gemm(codes8, scales8, w, sc, ex.scale2, workloads.NVFP4, out=out,
                                                       stream=stream),
    }
    for _ in range(args.warmup):
        for f in legs.values():
            f()
    torch.cuda.synchronize()
    K = args.steps
    us = {}
    for name, f in legs.items():
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        ev[0].record(stream)
        for i in range(K):
            f()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        us[name] = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(K)])) * 1e3
    flops = 2.0 * T * n * k
    tf = flops / (us["w4a4_gemm"] * 1e-6) / 1e12
    tf8 = flops / (us["fp4_expert_gemm"] * 1e-6) / 1e12
    log("  " + ", ".join(f"{nm} {u:.1f} us" for nm, u in us.items()))
    log(f"W4A4 GEMM {tf:.1f} TFLOP/s; FP8 x FP4 GEMM on the same shape {tf8:.1f} TFLOP/s")
    step_ms = (us["act_quant_fp4"] + us["w4a4_gemm"]) / 1e3
    result = {
        "metric": METRIC, "value": round(tf, 4), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp4xfp4->f32", "data": "synthetic",
        "config": {"workload": "w4a4: one NVFP4 expert n=4096 k=7168, 8192 tokens of 0.1 U[0,1), two-level E2M1",
                   "us": {nm: round(u, 2) for nm, u in us.items()}, "fp8_path_tflops": round(tf8, 1)},
        "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_PEAK_TFLOPS["f16"],
                     "unit": "TFLOP/s", "frac": round(tf / MFMA_PEAK_TFLOPS["f16"], 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

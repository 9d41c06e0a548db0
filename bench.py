#!/usr/bin/env python3
"""Benchmark of the MoE expert path on one MI355X.

One step = one whole MoE layer on one batch: [router logits] -> top-k routing
-> dispatch (plan + permutation) -> grouped GEMM1 + SwiGLU -> grouped GEMM2 ->
weighted combine, all through the library's C ABI on one HIP stream, inputs
resident in HBM.  The headline workload is the largest one-GPU configuration:
the DeepSeek-V3-shaped bf16 prefill layer with Zipf-skewed expert popularity
(T=8192 tokens, d_model=7168, d_ff=2048, 256 experts, top-8, sigmoid gates),
synthetic seeded inputs.  The other four workloads (tiny fp32 layer,
Mixtral-shaped prefill, DeepSeek-shaped decode, one expert-parallel rank's
share) are timed in the same run and reported under "others".  Prints ONE
JSON line.

Also reports, for the dominant pass (GEMM1 + SwiGLU), its achieved throughput
against the bound of its algorithmic work (HBM or bf16 MFMA), every pass's
roofline fraction, and the CPU oracle timed on a bounded sample of the
headline workload.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# CPU-baseline threading must be fixed before numpy loads its BLAS
_CORES = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_v, str(_CORES))

import numpy as np  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "MoE-layer tokens/s + TFLOP/s (MFMA %) and HBM GB/s (% peak), 1×MI355X"
HEADLINE = "dsv3_prefill_zipf"
# (the decode workload first: it shares the headline's expert weights)
OTHERS = ("dsv3_decode", "mixtral_prefill", "ep_rank_share", "tiny_fp32")
# workloads also timed with FP8 expert weights in the default run
FP8_WORKLOADS = ("dsv3_prefill_zipf", "dsv3_decode")
STEPS = ("router", "route", "dispatch", "ffn_up", "ffn_down", "combine")
DOMINANT = "ffn_up"                 # one GEMM1 + SwiGLU pass over all local rows
COPY_BYTES = 1 << 30

# kernels of each pass (substrings of the demangled names rocprofv3 reports)
PASS_KERNELS = {
    "router": ("router_logits_kernel", "router_logits_tiled_kernel"),
    "route": ("route_kernel", "route_candidates_kernel", "reroute_resolve_kernel",
              "reroute_finalize_kernel"),
    "dispatch_plan": ("dispatch_count_kernel", "dispatch_scan_kernel", "dispatch_place_kernel"),
    "permute": ("permute_rows_kernel",),
    "ffn_up": ("gemm_bf16_pipe<true", "gemm_bf16_kernel<32, 128, 64, 1, 4, true",
               "gemm_f32_kernel<true", "gemm_fp8_pipe<true", "gemm_fp8w_kernel<128, true"),
    "ffn_down": ("gemm_bf16_pipe<false", "gemm_bf16_kernel<32, 128, 64, 1, 4, false",
                 "gemm_f32_kernel<false", "gemm_fp8_pipe<false", "gemm_fp8w_kernel<128, false"),
    "combine": ("combine_kernel",),
}
# stored counter and kernel-time summaries are tied to the kernel sources
SOURCE_GLOBS = ("routing_dispatch_expert_moe_amd/csrc/*.hip", "routing_dispatch_expert_moe_amd/csrc/*.h",
                "routing_dispatch_expert_moe_amd/csrc/*.cpp")


def parse(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=HEADLINE)
    p.add_argument("--others", default=None,
                   help="comma-separated workloads timed after the headline one, or 'none' "
                        "(default: the other four when the headline is the default workload)")
    p.add_argument("--no-fused", action="store_true",
                   help="leave out the fused persistent launch (moe_forward_fused)")
    p.add_argument("--reroute", action="store_true",
                   help="route with capacity-overflow rerouting (moe_route_reroute)")
    p.add_argument("--weights", choices=("native", "fp8"), default="native",
                   help="fp8: quantise the packed bf16 expert weights to E4M3 codes with "
                        "128 x 128 block scales (moe_quantize_fp8, untimed) and run the FFN "
                        "steps on them")
    p.add_argument("--no-fp8", action="store_true",
                   help="leave out the FP8-weight runs of the DeepSeek-shaped workloads")
    p.add_argument("--backward", action="store_true",
                   help="also time a training step: the forward with the SwiGLU pre-activations "
                        "kept, then the whole backward pass (gradients of x, the gate logits "
                        "or router, and the expert weights); reported under 'training'")
    p.add_argument("--arrivals", type=int, default=0, metavar="S",
                   help="(a workload with a local expert range) also time the local expert FFN "
                        "on the rows that S source batches (seeds 0..S-1, each routed and "
                        "dispatched here) would send this rank: what one rank of an S-rank "
                        "expert-parallel layer computes; reported under 'arrivals'")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=64)
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (the counter calibration kernel)")
    p.add_argument("--traffic-from", default=None, metavar="DIR",
                   help="turn rocprofv3 --pmc databases under DIR/{fetch,write,copy_fetch,"
                        "copy_write} into profiles/traffic_<workload>.json and exit")
    p.add_argument("--counters-from", default=None, metavar="DIR",
                   help="summarise a rocprofv3 --pmc database under DIR taken with "
                        + " ".join(MFMA_COUNTERS) + " (MFMA busy fraction and counted "
                        "MFMA flops per kernel) and exit")
    p.add_argument("--trace-from", default=None, metavar="DIR",
                   help="summarise a rocprofv3 --kernel-trace run under DIR of this script "
                        "(--workload W --steps K --warmup W --others none --no-fused) into "
                        "profiles/kernels_<workload>.md and profiles/kernel_times_<workload>.json "
                        "and exit")
    p.add_argument("--profiles-dir", default=os.path.join(ROOT, "profiles"))
    return p.parse_args(argv)


def sources_hash():
    h = hashlib.sha256()
    for pat in SOURCE_GLOBS:
        for path in sorted(glob.glob(os.path.join(ROOT, pat))):
            h.update(os.path.basename(path).encode())
            with open(path, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def pass_of(kernel_name):
    for name, pats in PASS_KERNELS.items():
        if any(p in kernel_name for p in pats):
            return name
    return None


# ---- HBM traffic per pass from hardware counters --------------------------
#
# FETCH_SIZE and WRITE_SIZE (KiB per dispatch, summed over the channels) are
# taken in two rocprofv3 --pmc passes over a short bench run, and in two passes
# over a plain device copy of known size; the copy's counted bytes over its
# true bytes is the scale applied to the kernels' counts.  The result records a
# hash of the kernel sources: once they change, the stored traffic is stale
# and the bench reports null.

def copy_calibration():
    import torch
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 3}))


def _pmc_per_dispatch(path, counter):
    """{(db, dispatch_id): (kernel_name, value summed over dimensions)} from rocprofv3 databases."""
    import sqlite3
    out = {}
    files = glob.glob(os.path.join(path, "**", "*.db"), recursive=True)
    if not files:
        raise SystemExit(f"no rocprofv3 database under {path}")
    for f in files:
        con = sqlite3.connect(f)
        for did, kname, cname, val in con.execute(
                "select dispatch_id, kernel_name, counter_name, value from counters_collection"):
            if cname != counter:
                continue
            k = (f, did)
            name, v = out.get(k, (kname, 0.0))
            out[k] = (name, v + float(val))
    return out


# ---- MFMA utilisation of the MFMA kernels from hardware counters ------------
#
# One rocprofv3 --pmc pass with MFMA_COUNTERS over a short bench run.  As the
# database stores them, SQ_VALU_MFMA_BUSY_CYCLES is summed over every SIMD and
# GRBM_GUI_ACTIVE over the XCDs, so the busy fraction of the MFMA pipes while a
# kernel runs is busy / (GUI_ACTIVE / XCDs * SIMDs); SQ_INSTS_VALU_MFMA_MOPS_BF16
# counts MFMA work in units of 512 flops.
MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_BUSY_CYCLES",
                 "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_WAIT_INST_LDS", "SQ_INSTS_LDS",
                 "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE")
N_XCD, N_SIMD = 8, 256 * 4                      # MI355X: 8 XCDs, 256 CUs of 4 SIMDs


def counters_from(args):
    per = {}
    for ctr in MFMA_COUNTERS:
        for (f, did), (name, v) in _pmc_per_dispatch(args.counters_from, ctr).items():
            per.setdefault((f, did), {"kernel": name.split("(")[0]})[ctr] = v
    groups = {}
    for rec in per.values():
        if rec.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) > 0 and rec.get("GRBM_GUI_ACTIVE", 0) > 0:
            groups.setdefault(rec["kernel"], []).append(rec)
    for name, recs in sorted(groups.items(), key=lambda kv: -sum(r["SQ_VALU_MFMA_BUSY_CYCLES"]
                                                                 for r in kv[1])):
        mean = {c: float(np.mean([r.get(c, 0.0) for r in recs])) for c in MFMA_COUNTERS}
        cycles = mean["GRBM_GUI_ACTIVE"] / N_XCD
        print(json.dumps({
            "kernel": name, "dispatches": len(recs), "active_cycles": round(cycles),
            "mfma_busy_frac": round(mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * N_SIMD), 4),
            "mfma_flops_counted": mean["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512,
            "lds_bank_conflict_cycles": mean["SQ_LDS_BANK_CONFLICT"],
            "lds_instructions": mean["SQ_INSTS_LDS"],
            "lds_issue_wait_quad_cycles": mean["SQ_WAIT_INST_LDS"]}))


def traffic_from(args):
    """Counter bytes per call of every pass (each pass's kernels' mean counted
    KiB per dispatch, summed, scaled by the copy calibration)."""
    d = args.traffic_from
    scale = {}
    per_pass = {}
    for ctr, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        copy = [v for n, v in _pmc_per_dispatch(os.path.join(d, "copy_" + sub), ctr).values()
                if "copy" in n.lower() or "elementwise" in n.lower()]
        if not copy:
            raise SystemExit(f"{ctr}: no copy dispatches in the calibration run")
        copy_kib = float(np.median(copy))
        scale[ctr] = {"copy_counted_kib": copy_kib, "scale": (COPY_BYTES / 1024.0) / copy_kib}
        groups = {}
        for n, v in _pmc_per_dispatch(os.path.join(d, sub), ctr).values():
            p = pass_of(n)
            if p is not None:
                groups.setdefault(p, {}).setdefault(n.split("(")[0], []).append(v)
        for p, kern in groups.items():
            rec = per_pass.setdefault(p, {"kernels": {}})
            b = sum(float(np.mean(v)) for v in kern.values()) * 1024.0 * scale[ctr]["scale"]
            rec["fetch_bytes" if ctr == "FETCH_SIZE" else "write_bytes"] = b
            for kname, v in kern.items():
                rec["kernels"].setdefault(kname, {})[ctr + "_kib_per_dispatch"] = float(np.mean(v))
                rec["kernels"][kname]["dispatches"] = len(v)
    if DOMINANT not in per_pass:
        raise SystemExit("no dispatch of the dominant pass in the counter runs")
    for rec in per_pass.values():
        rec["bytes"] = rec.get("fetch_bytes", 0.0) + rec.get("write_bytes", 0.0)
    out = {"workload": args.workload, "sources_sha256_16": sources_hash(), "calibration": scale,
           "passes": per_pass}
    path = os.path.join(args.profiles_dir, f"traffic_{args.workload}.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps({p: round(r["bytes"]) for p, r in per_pass.items()}))


def load_stored(args, kind, workload):
    """profiles/<kind>_<workload>.json if it exists and matches the current
    kernel sources: (dict, note) or (None, reason)."""
    if getattr(args, "weights", "native") != "native":
        return None, "stored figures were taken with the native-precision weights"
    path = os.path.join(args.profiles_dir, f"{kind}_{workload}.json")
    if not os.path.exists(path):
        return None, f"no {os.path.basename(path)}"
    with open(path) as fh:
        t = json.load(fh)
    if t.get("workload") != workload:
        return None, "stored file is for another workload"
    if t.get("sources_sha256_16") != sources_hash():
        return None, "kernel sources changed since the stored figures were taken"
    return t, os.path.relpath(path, ROOT)


# ---- kernel-trace summary --------------------------------------------------

def _read_trace(d):
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *kernel_trace.csv under {d}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rd = csv.DictReader(fh)
            cols = {c.lower(): c for c in rd.fieldnames or []}
            kn, st, en = cols["kernel_name"], cols["start_timestamp"], cols["end_timestamp"]
            for r in rd:
                rows.append((int(r[st]), int(r[en]), r[kn]))
    rows.sort()
    return rows


def trace_from(args):
    """Per-kernel statistics of a profiled bench run and, per pass, the
    kernel time of each timed step (the run's dispatches of a pass are its
    warm-up steps, then the timed steps, then the cache-evicted steps).
    A run with --weights fp8 or --backward gets its own summary file
    (kernels_<workload>_fp8.md, kernels_training_<workload>.md) and no stored
    per-pass times (the forward passes' times are those of the native run;
    a training run's backward calls launch the same GEMM kernels)."""
    fp8 = getattr(args, "weights", "native") == "fp8"
    training = bool(getattr(args, "backward", False))
    forward_native = not (fp8 or training)
    rows = _read_trace(args.trace_from)
    stats = {}
    total = 0.0
    for s0, s1, n in rows:
        us = (s1 - s0) / 1e3
        total += us
        stats.setdefault(n.split("(")[0], []).append(us)
    per_pass = {}
    for s0, s1, n in rows:
        p = pass_of(n)
        if p is not None:
            per_pass.setdefault(p, []).append((s0, s1, n.split("(")[0]))
    W, K = args.warmup, args.steps
    passes = {}
    for p, disp in per_pass.items():
        names = sorted({n for _, _, n in disp})
        per_call = len(names)
        if len(disp) < (W + K) * per_call:
            continue
        timed = disp[W * per_call:(W + K) * per_call]
        steps = [sum((b - a) / 1e3 for a, b, _ in timed[i * per_call:(i + 1) * per_call])
                 for i in range(K)]
        passes[p] = {"kernels": names, "launches_per_call": per_call,
                     "per_step_us": [round(v, 2) for v in steps],
                     "mean_us": round(float(np.mean(steps)), 2)}
    event = None
    bl = os.path.join(args.trace_from, "bench.json")
    if os.path.exists(bl):
        with open(bl) as fh:
            event = json.loads(fh.read().strip().splitlines()[-1])
    out = {"workload": args.workload, "sources_sha256_16": sources_hash(), "steps": K,
           "warmup": W, "passes": passes}
    if event is not None:
        out["bench_event_mean_us"] = {p: round(v["ms"] * 1e3, 2)
                                      for p, v in event.get("per_step", {}).items()}
    if forward_native:
        with open(os.path.join(args.profiles_dir, f"kernel_times_{args.workload}.json"), "w") as fh:
            json.dump(out, fh, indent=1)
    extra = (" --weights fp8" if fp8 else "") + (" --backward" if training else "")
    cmd = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv "
           f"-d <out> -o kt -- python3 <repo>/bench.py --workload {args.workload}{extra} --steps {K} "
           f"--warmup {W} --others none --no-fused --no-cpu-baseline > <out>/bench.json")
    what = ("MoE training step (forward + backward)" if training else "MoE layer") + \
        (", FP8 (E4M3) expert weights" if fp8 else "")
    runs = (f"{W} warm-up and {K} timed layer steps of the separate calls, then {K} more with the "
            "Infinity Cache evicted before each (a 1 GiB fill between steps), then the "
            "dispatch plan alone, then five 1 GiB copies (the bench's plain-copy reference)")
    if fp8:
        runs += "; the weights are quantised once first (`moe_quantize_fp8`)"
    if training:
        runs += (f"; then {W} warm-up and {K} timed training steps (the forward with the "
                 "pre-activations kept, then the backward calls)")
    lines = [f"# Kernel time summary: {what}, workload {args.workload}", "",
             "Command (from the repository root, on one MI355X):", "", "    " + cmd, "",
             runs + ".  Weight packing and input upload run once before them.  Durations are "
             "the kernel trace's start/end stamps, in microseconds.", "",
             "| kernel | calls | avg us | min us | max us | % of traced GPU time |",
             "|---|---|---|---|---|---|"]
    for n, v in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{n}` | {len(v)} | {np.mean(v):.2f} | {min(v):.2f} | {max(v):.2f} | "
                     f"{100 * sum(v) / total:.2f} |")
    if training:
        passes = {}  # the backward launches the forward's GEMM kernels too
    else:
        lines += ["", "Per pass, kernel time of each timed step (sum over the pass's kernels):", "",
                  "| pass | kernels | per-step us | mean us | bench HIP-event mean us |",
                  "|---|---|---|---|---|"]
    for p in ("router", "route", "dispatch_plan", "permute", "ffn_up", "ffn_down", "combine"):
        if p in passes:
            r = passes[p]
            ev = (out.get("bench_event_mean_us") or {}).get(p, "")
            lines.append(f"| {p} | {', '.join('`' + k + '`' for k in r['kernels'])} | "
                         f"{', '.join(f'{v:.1f}' for v in r['per_step_us'])} | {r['mean_us']:.1f} | "
                         f"{ev} |")
    lines.append("")
    name = ("training_" if training else "") + args.workload + ("_fp8" if fp8 else "")
    with open(os.path.join(args.profiles_dir, f"kernels_{name}.md"), "w") as fh:
        fh.write("\n".join(lines))
    print(json.dumps({p: r["mean_us"] for p, r in passes.items()}))


# ---- the benchmark ----------------------------------------------------------

def smi_snapshot():
    """Graphics and memory clocks and socket power read from the driver's sysfs
    files (plain reads; no program is started): {"sclk_mhz", "mclk_mhz",
    "socket_power_w", "power_cap_w"}, or None where they are missing."""
    import re

    def current(path):
        with open(path) as fh:
            for line in fh:
                if line.rstrip().endswith("*"):
                    m = re.search(r"(\d+)\s*Mhz", line, re.I)
                    return int(m.group(1)) if m else None
        return None

    try:
        dev = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))[0].rsplit("/", 1)[0]
        out = {"sclk_mhz": current(dev + "/pp_dpm_sclk"), "mclk_mhz": current(dev + "/pp_dpm_mclk")}
        hw = sorted(glob.glob(dev + "/hwmon/hwmon*"))
        if hw:
            for key, name in (("socket_power_w", "power1_input"), ("power_cap_w", "power1_cap")):
                try:
                    with open(f"{hw[0]}/{name}") as fh:
                        out[key] = round(int(fh.read().strip()) / 1e6, 1)
                except (OSError, ValueError):
                    out[key] = None
        return out
    except (IndexError, OSError):
        return None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def bf16_dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def work_model(wl, n, touched, T_read, wb=None):
    """Algorithmic flops and HBM bytes per launch of each step (wb: bytes per
    weight element when it differs from the activations', e.g. 1 for FP8
    codes; their block scales add 4 B per 128 x 128 block).  'dispatch' is the
    whole call; 'dispatch_plan' and 'permute' are its two parts."""
    b = 2 if wl.dtype == "bf16" else 4
    if wb is None:
        wb = b
    T, d, f, E, k = wl.T, wl.d, wl.f, wl.E, wl.k
    m = {
        "router": (2.0 * T * d * E if wl.w_gate is not None else 0.0,
                   (T * d * b + d * E * 4 + T * E * 4) if wl.w_gate is not None else 0.0),
        "route": (0.0, T * E * 4 + T * k * 8),
        "dispatch_plan": (0.0, 12.0 * T * k),
        "permute": (0.0, T_read * d * b + n * d * b),
        "ffn_up": (4.0 * n * d * f, touched * 2.0 * f * d * wb + n * d * b + n * f * b),
        "ffn_down": (2.0 * n * f * d, touched * 1.0 * d * f * wb + n * f * b + n * d * b),
        "combine": (0.0, n * d * b + T * k * 8 + T * d * b),
    }
    m["dispatch"] = (0.0, m["dispatch_plan"][1] + m["permute"][1])
    return m


def roofline_of(fl, by, ms):
    """The pass's bound (whichever of its algorithmic flops at the bf16 MFMA peak
    and its algorithmic bytes at the HBM peak takes longer) and the fraction
    of that bound's time its measured time reaches."""
    t_mfma = fl / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = by / (PEAK_HBM_GBS * 1e9)
    if ms <= 0 or (t_mfma == 0 and t_hbm == 0):
        return None
    if t_mfma >= t_hbm:
        return {"bound": "mfma", "achieved": round(fl / (ms * 1e-3) / 1e12, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(t_mfma / (ms * 1e-3), 4)}
    return {"bound": "hbm", "achieved": round(by / (ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(t_hbm / (ms * 1e-3), 4)}


def cpu_baseline(wl, host_w, n_tok):
    """The CPU oracle (float64) on the first n_tok tokens of the workload, grown once
    so that a pass takes seconds; when the whole workload is that fast, passes are
    repeated until about 10 s of CPU work has been timed.  Returns (tokens/s,
    seconds timed, tokens per pass, passes)."""
    rate, dt = _cpu_oracle(wl, host_w, n_tok)
    if dt < 8.0 and n_tok < wl.T:
        n_tok = min(wl.T, int(n_tok * 15.0 / max(dt, 1e-3)))
        rate, dt = _cpu_oracle(wl, host_w, n_tok)
    total, passes = dt, 1
    while total < 10.0 and passes < 8:
        _, dt = _cpu_oracle(wl, host_w, n_tok)
        total += dt
        passes += 1
    return n_tok * passes / total, total, n_tok, passes


def _cpu_oracle(wl, host_w, n_tok):
    from oracle import moe_oracle as O
    x = wl.x[:n_tok]
    t0 = time.perf_counter()
    x64 = O.widen(x, wl.dtype)
    if wl.w_gate is not None:
        logits = O.round_to_f32(O.router_logits(x64, wl.w_gate.astype(np.float64)))
    else:
        logits = wl.logits[:n_tok]
    C = O.capacity(n_tok, wl.k, wl.E, wl.capacity_factor)
    out = O.moe_layer(x, wl.dtype, logits, wl.k, wl.gate,
                      lambda i: tuple(O.widen(a, wl.dtype) for a in host_w[i]), wl.E, C,
                      wl.e_begin, wl.e_end)
    dt = time.perf_counter() - t0
    assert out["y"].shape == (n_tok, wl.d)
    return n_tok / dt, dt


TRAIN_STEPS = ("router", "route", "dispatch", "ffn_up_train", "ffn_down", "combine",
               "combine_bwd", "gate_bwd", "ffn_down_bwd", "ffn_up_bwd", "combine_dx",
               "router_bwd", "wgrad")


def train_work_model(wl, n, touched, T_read):
    """Algorithmic flops and bytes of each call of a training step."""
    b = 2 if wl.dtype == "bf16" else 4
    T, d, f, E, k = wl.T, wl.d, wl.f, wl.E, wl.k
    m = work_model(wl, n, touched, T_read)
    m["ffn_up_train"] = (m["ffn_up"][0], m["ffn_up"][1] + 2.0 * n * f * b)
    router = wl.w_gate is not None
    m.update({
        "combine_bwd": (2.0 * n * d, T * d * b + 2.0 * n * d * b + T * k * 12),
        "gate_bwd": (0.0, T * E * 4 + T * k * 12),
        # dh = do W2^T, then SwiGLU' from the saved pre-activations
        "ffn_down_bwd": (2.0 * n * d * f, touched * 1.0 * f * d * b + n * d * b + 2.0 * n * f * b
                         + 4.0 * n * f * b),
        "ffn_up_bwd": (4.0 * n * d * f, touched * 2.0 * f * d * b + 2.0 * n * f * b + n * d * b),
        "combine_dx": (0.0, n * d * b + T * d * b),
        "router_bwd": ((4.0 * T * d * E, 3.0 * T * d * b + d * E * 8 + T * E * 4) if router
                       else (0.0, 0.0)),
        # dW13 = dab^T x_perm, dW2 = do^T h: read the four operands, write fp32 gradients
        "wgrad": (6.0 * n * d * f, n * (2 * d + 3 * f) * b + touched * 3.0 * d * f * 4),
    })
    return m


def train_bench(args, wl, layer, x, logits, wg, w13_t, w2_t, n, touched, T_read, dev):
    """Time training steps (forward with saved pre-activations + backward) with
    HIP events around every call; returns the 'training' object."""
    import torch
    from workloads import output_grad
    layer.enable_training(w13_t, w2_t)
    dy = (bf16_dev(output_grad(wl), dev) if wl.dtype == "bf16"
          else torch.from_numpy(output_grad(wl)).to(dev))
    router = wg is not None

    def tstep(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        lg = layer.router(x, wg) if router else logits
        mark(1)
        layer.route(lg)
        mark(2)
        layer.dispatch(x)
        mark(3)
        layer.ffn_up_train()
        mark(4)
        layer.ffn_down()
        mark(5)
        layer.combine()
        mark(6)
        layer.combine_backward(dy)
        mark(7)
        layer.gate_backward(lg)
        mark(8)
        layer.ffn_down_backward()
        mark(9)
        layer.ffn_up_backward()
        mark(10)
        layer.combine_dx()
        mark(11)
        if router:
            layer.router_backward(x, wg)
        mark(12)
        layer.wgrad()
        mark(13)

    import routing_dispatch_expert_moe_amd as M
    for _ in range(args.warmup):
        tstep()
    torch.cuda.synchronize()
    if M.moe_check_error(layer.ws) != 0:
        raise RuntimeError("device error in the training step")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(14)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        tstep(ev[s])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    model = train_work_model(wl, n, touched, T_read)
    per = {}
    for i, name in enumerate(TRAIN_STEPS):
        ms = float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)]))
        fl, by = model[name]
        per[name] = {"ms": round(ms, 5),
                     "tflops": round(fl / (ms * 1e-3) / 1e12, 2) if fl and ms > 0 else None,
                     "gbs": round(by / (ms * 1e-3) / 1e9, 1) if by and ms > 0 else None}
    bwd_ms = float(np.mean([ev[s][6].elapsed_time(ev[s][13]) for s in range(args.steps)]))
    fl = sum(model[k][0] for k in TRAIN_STEPS)
    # the dominant backward call: the longest one
    dom = max(TRAIN_STEPS[6:], key=lambda k: per[k]["ms"])
    dfl, dby = model[dom]
    dms = per[dom]["ms"]
    roof = roofline_of(dfl, dby, dms)
    roof.update(call=dom, avg_launch_ms=dms, algorithmic_flops_per_launch=dfl,
                algorithmic_bytes_per_launch=dby)
    return {"ms_per_step": round(ms_step, 4), "tokens_per_s": round(wl.T / (ms_step * 1e-3), 1),
            "backward_ms": round(bwd_ms, 4), "step_tflops": round(fl / (ms_step * 1e-3) / 1e12, 2),
            "per_call": per, "roofline": roof,
            "note": "one step = forward (pre-activations kept) + backward: combine, gate and "
                    "router backward, dh and SwiGLU', dx, fp32 weight gradients; HIP events "
                    "around every call on the launch stream"}


class Weights:
    """Packed device weights of the workloads, generated on the host once per
    weight set (the DeepSeek-shaped decode and prefill workloads share theirs)."""

    def __init__(self, dev):
        self.dev = dev
        self.key = None
        self.val = None

    def get(self, wl, keep_host=False, train=False):
        import torch
        import routing_dispatch_expert_moe_amd as M
        key = (wl.E_loc, wl.e_begin, wl.d, wl.f, wl.seed, wl.dtype)
        if (self.key == key and (not keep_host or self.val[2] is not None)
                and (not train or self.val[3] is not None)):
            return self.val
        self.key = self.val = None
        torch.cuda.empty_cache()
        dev = self.dev
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        w13 = torch.empty((wl.E_loc, 2 * wl.f, wl.d), dtype=tdt, device=dev)
        w2p = torch.empty((wl.E_loc, wl.d, wl.f), dtype=tdt, device=dev)
        host_w = [] if keep_host else None
        w13_t = w2_t = None
        if train:   # the backward operands: [W1 | W3] rows per d, and W2 as it is
            w13_t = torch.empty((wl.E_loc, wl.d, 2 * wl.f), dtype=tdt, device=dev)
            w2_t = torch.empty((wl.E_loc, wl.f, wl.d), dtype=tdt, device=dev)

        def up(a):
            return bf16_dev(a, dev) if wl.dtype == "bf16" else torch.from_numpy(a).to(dev)

        for c0 in range(0, wl.E_loc, 16):
            ids = list(range(wl.e_begin + c0, wl.e_begin + min(wl.E_loc, c0 + 16)))
            a, b, c = wl.stacked_weights(ids)
            if keep_host:
                host_w.extend(zip(a, b, c))
            ga, gb, gc = up(a), up(b), up(c)
            M.moe_pack_weights(ga, gb, gc, w13[c0:c0 + len(ids)], w2p[c0:c0 + len(ids)])
            if train:
                M.moe_pack_weights_backward(ga, gb, w13_t[c0:c0 + len(ids)])
                w2_t[c0:c0 + len(ids)] = gc
            del ga, gb, gc
        torch.cuda.synchronize()
        self.key, self.val = key, (w13, w2p, host_w, w13_t, w2_t)
        return self.val


def run_workload(args, wl, weights, dev, headline, fp8=None):
    """Time one workload's layer: K steps of the separate calls (HIP events
    around each call), the same steps with the Infinity Cache evicted, the
    dispatch plan alone, and the fused launch; returns the results dict."""
    import torch
    import routing_dispatch_expert_moe_amd as M

    log(f"workload {wl.name}: T={wl.T} d={wl.d} f={wl.f} E={wl.E} k={wl.k} dtype={wl.dtype}")
    train = headline and args.backward
    keep_host = headline and not args.no_cpu_baseline
    w13, w2p, host_w, w13_t, w2_t = weights.get(wl, keep_host=keep_host, train=train)
    log("weights packed")
    C = M.moe_capacity(wl.T, wl.k, wl.E, wl.capacity_factor)
    if fp8 is None:
        fp8 = headline and args.weights == "fp8"
    reroute = headline and args.reroute
    s13 = s2 = None
    if fp8:
        if wl.dtype != "bf16":
            raise SystemExit("--weights fp8 needs a bf16 workload")
        q13, s13 = M.moe_quantize_fp8(w13)
        q2, s2 = M.moe_quantize_fp8(w2p)
        torch.cuda.synchronize()
        w13, w2p = q13, q2
        log("weights quantised to E4M3 with 128 x 128 block scales")
    layer = M.MoELayer(w13, w2p, E=wl.E, k=wl.k, gate=wl.gate, T=wl.T, capacity=C,
                       w13_scale=s13, w2_scale=s2, reroute=reroute,
                       e_begin=wl.e_begin, e_end=wl.e_end)
    x = bf16_dev(wl.x, dev) if wl.dtype == "bf16" else torch.from_numpy(wl.x).to(dev)
    logits = torch.from_numpy(wl.logits).to(dev) if wl.logits is not None else None
    wg = torch.from_numpy(wl.w_gate).to(dev) if wl.w_gate is not None else None

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        lg = layer.router(x, wg) if wg is not None else logits
        if ev is not None:
            ev[1].record()
        layer.route(lg)
        if ev is not None:
            ev[2].record()
        layer.dispatch(x)
        if ev is not None:
            ev[3].record()
        layer.ffn_up()
        if ev is not None:
            ev[4].record()
        layer.ffn_down()
        if ev is not None:
            ev[5].record()
        layer.combine()
        if ev is not None:
            ev[6].record()

    K = args.steps
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    status = M.moe_check_error(layer.ws)
    if status != 0:
        raise RuntimeError(f"device error {status}")
    n = int(layer.plan.n_kept[0].item())
    counts = layer.plan.counts.cpu().numpy()[wl.e_begin:wl.e_end]
    kept = np.minimum(counts, C) if C >= 0 else counts
    touched = int((kept > 0).sum())
    pp = layer.plan.pair_pos.cpu().numpy()[:wl.T * wl.k].reshape(wl.T, wl.k)
    T_read = int((pp >= 0).any(axis=1).sum())
    log(f"n_kept={n} experts touched={touched} rows per expert min={kept.min()} max={kept.max()}")

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(K)]
    smi_before = smi_snapshot() if headline else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        step(events[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    smi_after = smi_snapshot() if headline else None
    ms_step = (t1 - t0) * 1e3 / K

    # the same steps with the 256 MB Infinity Cache (MALL) evicted before each:
    # a 1 GiB write between steps, outside the events, so that no step starts
    # with its inputs or weights cache-resident (per-step HIP-event times)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cev = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(K)]
    for s in range(K):
        scratch.fill_(s & 0xFF)
        step(cev[s])
    # the dispatch plan alone (no permutation), so the permutation's own time
    # is the dispatch call's minus this
    pev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for s in range(K):
        pev[s][0].record()
        M.moe_dispatch(layer.topk_idx, wl.E, C, wl.e_begin, wl.e_end, None, layer.ws,
                       layer.plan, d=layer.d, dtype=layer.dtype)
        pev[s][1].record()
    torch.cuda.synchronize()
    copy_ms = None
    if headline:
        # a plain-copy reference on the same device and under the same eviction:
        # torch's copy_ of a 1 GiB buffer, read + write bytes counted
        src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        rev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(5)]
        for s in range(5):
            scratch.fill_(s)
            rev[s][0].record()
            dst.copy_(src)
            rev[s][1].record()
        torch.cuda.synchronize()
        copy_ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in rev]))
        del src, dst
    del scratch
    cold_ms = {name: float(np.median([cev[s][i].elapsed_time(cev[s][i + 1]) for s in range(K)]))
               for i, name in enumerate(STEPS)}
    cold_step = float(np.median([cev[s][0].elapsed_time(cev[s][6]) for s in range(K)]))
    plan_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in pev]))

    # the same layer as one fused persistent launch (router logits stay a separate call)
    fused_ms = None
    fused_orders = None
    # (FP8 weights: moe_forward_fused_fp8, which routes without rerouting)
    if not (args.no_fused or (fp8 and reroute)):
        fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]

        def fused_step(ev=None):
            if ev is not None:
                ev[0].record()
            lg = layer.router(x, wg) if wg is not None else logits
            layer.forward_fused(x, lg)
            if ev is not None:
                ev[1].record()
        def time_fused():
            for _ in range(args.warmup):
                fused_step()
            torch.cuda.synchronize()
            for s in range(K):
                fused_step(fev[s])
            torch.cuda.synchronize()
            if M.moe_check_error(layer.ws) != 0:
                raise RuntimeError("device error in the fused layer")
            return float(np.median([e[0].elapsed_time(e[1]) for e in fev]))
        fused_ms = time_fused()  # the library's own choice of GEMM-phase order
        # both orders of the two GEMM phases, forced: a device-wide barrier
        # between them, and per-expert waits (where possible)
        fused_orders = {}
        try:
            for mode in ("never", "always"):
                M.moe_set_fused_overlap(mode)
                fused_orders[mode] = time_fused()
        finally:
            M.moe_set_fused_overlap("auto")
    unfused_ms = float(np.median([events[s][0].elapsed_time(events[s][6]) for s in range(K)]))

    model = work_model(wl, n, touched, T_read, wb=(1 + 4.0 / (128 * 128)) if fp8 else None)
    per = {}
    for i, name in enumerate(STEPS):
        ms = float(np.mean([events[s][i].elapsed_time(events[s][i + 1]) for s in range(K)]))
        per[name] = {"ms": round(ms, 5)}
    per["dispatch_plan"] = {"ms": round(plan_ms, 5)}
    per["permute"] = {"ms": round(max(per["dispatch"]["ms"] - plan_ms, 0.0), 5),
                      "note": "dispatch call minus the plan alone"}
    for name, rec in per.items():
        fl, by = model[name]
        ms = rec["ms"]
        rec["tflops"] = round(fl / (ms * 1e-3) / 1e12, 2) if fl and ms > 0 else None
        rec["gbs"] = round(by / (ms * 1e-3) / 1e9, 1) if by and ms > 0 else None
        rec["roofline"] = roofline_of(fl, by, ms) if (fl or by) else None
    cold = {name: {"ms": round(ms, 5),
                   "gbs": round(model[name][1] / (ms * 1e-3) / 1e9, 1) if model[name][1] else None}
            for name, ms in cold_ms.items()}
    flops = sum(model[k][0] for k in STEPS)
    bytes_ = sum(model[k][1] for k in STEPS)
    plan_code = M.moe_ffn_plan("up", layer.plan.max_rows, wl.E_loc, wl.d, wl.f,
                               dtype=wl.dtype, cu_count=torch.cuda.get_device_properties(dev)
                               .multi_processor_count) if not fp8 else "fp8"
    res = {"wl": wl, "layer": layer, "x": x, "logits": logits, "wg": wg, "host_w": host_w,
           "w13_t": w13_t, "w2_t": w2_t, "n": n, "touched": touched, "T_read": T_read, "C": C,
           "ms_step": ms_step, "per": per, "cold": cold, "cold_step": cold_step,
           "fused_ms": fused_ms, "fused_orders": fused_orders, "unfused_ms": unfused_ms, "model": model, "flops": flops,
           "bytes": bytes_, "copy_ms": copy_ms, "smi": (smi_before, smi_after), "fp8": fp8,
           "reroute": reroute, "plan_up": plan_code,
           "rows_per_expert": [int(kept.min()), int(kept.max())]}
    return res


def dominant_roofline(args, r):
    """The roofline object of the dominant pass (GEMM1 + SwiGLU)."""
    wl = r["wl"]
    fl, by = r["model"][DOMINANT]
    ms = r["per"][DOMINANT]["ms"]
    roof = roofline_of(fl, by, ms)
    kernels = {"f32": "gemm_f32_kernel<SwiGLU>", "stream": "gemm_bf16_kernel<32-row tiles, SwiGLU>",
               "wide": "gemm_bf16_pipe<SwiGLU, 128-row tiles>",
               "big_all": "gemm_bf16_pipe<SwiGLU, 256-row tiles>",
               "big_tail": "gemm_bf16_pipe<SwiGLU, 256-row tiles> + 128-row remainder tiles",
               "big_ride": "gemm_bf16_pipe<SwiGLU, 256-row tiles> + 128-row tiles (experts < 128 rows)",
               "fp8": "FP8-weight GEMM1 + SwiGLU"}
    roof["kernel"] = f"{DOMINANT}: " + kernels.get(r["plan_up"], r["plan_up"])
    roof["algorithmic_flops_per_launch"] = fl
    roof["algorithmic_bytes_per_launch"] = by
    roof["avg_launch_ms"] = ms
    roof["timing"] = "HIP events on the launch stream around each call, mean over the timed steps"
    tr, note = load_stored(args, "traffic", wl.name)
    if tr is not None and r["fp8"] is False:
        roof["traffic"] = round(tr["passes"][DOMINANT]["bytes"])
        roof["traffic_note"] = f"rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a 1 GiB copy ({note})"
    else:
        roof["traffic"] = None
        roof["traffic_note"] = note
    kt, note = load_stored(args, "kernel_times", wl.name)
    if kt is not None and DOMINANT in kt["passes"]:
        pm = kt["passes"][DOMINANT]["mean_us"] * 1e-3
        pr = roofline_of(fl, by, pm)
        roof["profile"] = {"avg_launch_ms": round(pm, 5), "achieved": pr["achieved"],
                           "frac": pr["frac"], "file": note.replace("kernel_times_", "kernels_")
                           .replace(".json", ".md"),
                           "note": "kernel-trace duration of the pass per timed step in a "
                                   "rocprofv3 run of the same sources (another run, maybe "
                                   "another box)"}
    else:
        roof["profile"] = None
        roof["profile_note"] = note
    return roof


def traffic_per_pass(args, r):
    tr, note = load_stored(args, "traffic", r["wl"].name)
    if tr is None or r["fp8"]:
        return None
    out = {}
    for p, rec in tr["passes"].items():
        alg = r["model"].get(p, (0, 0))[1]
        out[p] = {"counter_bytes": round(rec["bytes"]), "algorithmic_bytes": round(alg),
                  "counter_over_algorithmic": round(rec["bytes"] / alg, 3) if alg else None}
    return {"passes": out, "source": note}


def summary_of(args, r):
    """The compact record of a non-headline workload."""
    wl = r["wl"]
    out = {"workload": wl.name, "tokens": wl.T, "d_model": wl.d, "d_ff": wl.f, "experts": wl.E,
           "local_experts": wl.E_loc, "top_k": wl.k, "dtype": wl.dtype, "capacity": r["C"],
           "n_kept": r["n"], "rows_per_expert_min_max": r["rows_per_expert"],
           "ms_per_step": round(r["ms_step"], 4),
           "tokens_per_s": round(wl.T / (r["ms_step"] * 1e-3), 1),
           "layer_tflops": round(r["flops"] / (r["ms_step"] * 1e-3) / 1e12, 2),
           "layer_hbm_gbs": round(r["bytes"] / (r["ms_step"] * 1e-3) / 1e9, 1),
           "per_step": r["per"], "mall_flushed_ms_per_step": round(r["cold_step"], 4),
           "roofline": dominant_roofline(args, r), "traffic_per_pass": traffic_per_pass(args, r)}
    if r["fused_ms"] is not None:
        out["fused"] = {"ms_per_step_median": round(r["fused_ms"], 4),
                        "unfused_ms_per_step_median": round(r["unfused_ms"], 4),
                        "speedup_vs_unfused": round(r["unfused_ms"] / r["fused_ms"], 3),
                        **fused_orders_out(r)}
    return out


def fused_orders_out(r):
    """The fused launch's time with each order of its GEMM phases forced."""
    o = r.get("fused_orders")
    if not o:
        return {}
    return {"barrier_ms_per_step_median": round(o["never"], 4),
            "overlap_ms_per_step_median": round(o["always"], 4),
            "orders_note": "moe_set_fused_overlap forced: a device-wide barrier between the "
                           "GEMM phases, then per-expert waits; ms_per_step_median is the "
                           "library's automatic choice"}


def join_arrivals(parts, E_loc):
    """The rows one rank receives from several sources, as its FFN takes them:
    parts[s] = (x_perm of source s, its local offsets list); the result holds
    expert 0's rows of source 0, then of source 1, ..., then expert 1's, and
    the joined offsets (E_loc + 1 ints)."""
    import torch
    segs, offsets = [], [0]
    for i in range(E_loc):
        for xp, off in parts:
            if off[i + 1] > off[i]:
                segs.append(xp[off[i]:off[i + 1]])
        offsets.append(offsets[-1] + sum(off[i + 1] - off[i] for _, off in parts))
    xp0 = parts[0][0]
    x_perm = torch.cat(segs) if segs else torch.zeros((1, xp0.shape[1]), dtype=xp0.dtype,
                                                      device=xp0.device)
    return x_perm, offsets


def arrivals_bench(args, name, weights, dev):
    """The local expert FFN at the load one rank of an S-rank expert-parallel
    layer receives: S seeded source batches of the workload (its x and logits
    from seeds 0..S-1; the rank's local experts' weights from seed 0) are each
    routed and dispatched here with the workload's capacity and local range,
    and their kept rows are joined expert by expert, source by source (what
    the receive side of the exchange would hold).  The join runs once,
    untimed; K steps of the two FFN halves on the joined rows are timed with
    HIP events."""
    import torch
    import routing_dispatch_expert_moe_amd as M
    from workloads import make

    S = args.arrivals
    wl0 = make(name)
    if wl0.E_loc == wl0.E:
        raise SystemExit("--arrivals needs a workload with a local expert range")
    w13, w2p, _, _, _ = weights.get(wl0)
    C = M.moe_capacity(wl0.T, wl0.k, wl0.E, wl0.capacity_factor)
    parts = []
    for src in range(S):
        ws_ = make(name, seed=src)
        layer = M.MoELayer(w13, w2p, E=ws_.E, k=ws_.k, gate=ws_.gate, T=ws_.T, capacity=C,
                           e_begin=ws_.e_begin, e_end=ws_.e_end)
        layer.route(torch.from_numpy(ws_.logits).to(dev))
        layer.dispatch(bf16_dev(ws_.x, dev))
        torch.cuda.synchronize()
        if M.moe_check_error(layer.ws) != 0:
            raise RuntimeError("device error in an arrivals source batch")
        off = layer.plan.offsets.cpu().tolist()
        parts.append((layer.plan.x_perm, off))
        del layer
    E_loc = wl0.E_loc
    x_perm, offsets = join_arrivals(parts, E_loc)
    n = offsets[-1]
    del parts
    off_t = torch.tensor(offsets, dtype=torch.int32, device=dev)
    rows = max(n, 1)
    h = torch.empty((rows, wl0.f), dtype=torch.bfloat16, device=dev)
    y = torch.empty((rows, wl0.d), dtype=torch.bfloat16, device=dev)
    for _ in range(args.warmup):
        M.moe_ffn_up(x_perm, off_t, E_loc, n, w13, h)
        M.moe_ffn_down(h, off_t, E_loc, n, w2p, y)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e3 in ev:
        e3[0].record()
        M.moe_ffn_up(x_perm, off_t, E_loc, n, w13, h)
        e3[1].record()
        M.moe_ffn_down(h, off_t, E_loc, n, w2p, y)
        e3[2].record()
    torch.cuda.synchronize()
    up = sum(e3[0].elapsed_time(e3[1]) for e3 in ev) / len(ev)
    down = sum(e3[1].elapsed_time(e3[2]) for e3 in ev) / len(ev)
    per = [offsets[i + 1] - offsets[i] for i in range(E_loc)]
    touched = sum(1 for r in per if r > 0)
    m = work_model(wl0, n, touched, 0)
    out = {"sources": S, "rows": n, "rows_per_expert_min_max": [min(per), max(per)],
           "capacity_per_source": C, "ms_ffn": round(up + down, 4),
           "rows_per_s": round(n / ((up + down) * 1e-3), 1)}
    for key, ms in (("ffn_up", up), ("ffn_down", down)):
        fl, by = m[key]
        out[key] = {"ms": round(ms, 5), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                    "gbs": round(by / (ms * 1e-3) / 1e9, 1), "roofline": roofline_of(fl, by, ms)}
    out["note"] = ("x and logits of seeds 0..S-1 routed and dispatched on this GPU, kept local "
                   "rows joined per expert (untimed); HIP events around each FFN half")
    return out


def main(argv=None):
    args = parse(argv)
    if args.traffic_from:
        traffic_from(args)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.counters_from:
        counters_from(args)
        return
    if args.trace_from:
        trace_from(args)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; "
                                   f"--gpus {args.gpus} is not supported (the path is single-GPU)"}))
        sys.exit(2)
    import torch
    from workloads import make

    dev = torch.device("cuda:0")
    if args.others is None:
        others = list(OTHERS) if args.workload == HEADLINE else []
    elif args.others == "none":
        others = []
    else:
        others = [w for w in args.others.split(",") if w and w != args.workload]
    weights = Weights(dev)
    wl = make(args.workload)
    r = run_workload(args, wl, weights, dev, headline=True)
    ms_step = r["ms_step"]
    roofline = dominant_roofline(args, r)

    training = None
    if args.backward:
        if r["fp8"] or args.reroute:
            raise SystemExit("--backward takes native weights and plain top-k routing")
        training = train_bench(args, wl, r["layer"], r["x"], r["logits"], r["wg"], r["w13_t"],
                               r["w2_t"], r["n"], r["touched"], r["T_read"], dev)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle on {args.cpu_sample_tokens} tokens")
        rate, dt, n_tok, passes = cpu_baseline(wl, r["host_w"], args.cpu_sample_tokens)
        cpu = {"value": round(rate, 2), "unit": "tokens/s", "cores": _CORES, "kind": "oracle",
               "sample": f"first {n_tok} of {wl.T} tokens of {wl.name} (capacity rule applied "
                         f"to the sample), whole layer in float64 (router..combine), "
                         f"{passes} pass(es), {dt:.1f} s timed"}
    head_summary = {k: r[k] for k in ("fused_ms", "unfused_ms")}
    head_orders = fused_orders_out(r)
    smi_before, smi_after = r["smi"]
    copy_ms = r["copy_ms"]
    tflops = r["flops"] / (ms_step * 1e-3) / 1e12
    gbs = r["bytes"] / (ms_step * 1e-3) / 1e9
    line = {
        "metric": METRIC, "value": round(wl.T / (ms_step * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": wl.name, "tokens": wl.T, "d_model": wl.d, "d_ff": wl.f,
                   "experts": wl.E, "local_experts": wl.E_loc, "top_k": wl.k, "gate": wl.gate,
                   "capacity": r["C"], "parallelism": "single GPU",
                   "weights": "e4m3 codes, fp32 scale per 128x128 block" if r["fp8"] else wl.dtype,
                   "routing": "top-k with overflow rerouting" if r["reroute"] else "top-k",
                   "rows_per_expert_min_max": r["rows_per_expert"], "n_kept": r["n"]},
        "layer_tflops": round(tflops, 2), "layer_mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "layer_hbm_gbs": round(gbs, 1), "layer_hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "per_step": r["per"], "roofline": roofline, "traffic_per_pass": traffic_per_pass(args, r),
        "cpu_baseline": cpu,
        "mall_flushed": {"ms_per_step_median": round(r["cold_step"], 4),
                         "per_step_median": r["cold"],
                         "note": "1 GiB written between steps (outside the events) to evict "
                                 "the 256 MB Infinity Cache; HIP-event times per call"},
        "hbm_copy_reference": {"gbs": round(2 * COPY_BYTES / (copy_ms * 1e-3) / 1e9, 1),
                               "frac_of_peak": round(2 * COPY_BYTES / (copy_ms * 1e-3) / 1e9
                                                     / PEAK_HBM_GBS, 4),
                               "note": "torch copy_ of a 1 GiB buffer (read + write bytes), "
                                       "Infinity Cache evicted before each, median of 5: "
                                       "what a plain copy reaches on this device"},
        "power_clock": {"before_timed_steps": smi_before, "after_timed_steps": smi_after,
                        "note": "driver sysfs snapshots (current graphics and memory clock "
                                "levels, socket power) just before and just after the timed "
                                "steps"},
        "training": training,
        "fused": None if head_summary["fused_ms"] is None else {
            "entry": ("moe_forward_fused_reroute" if r["reroute"] else
                      "moe_forward_fused_fp8" if r["fp8"] else "moe_forward_fused"),
            "ms_per_step_median": round(head_summary["fused_ms"], 4),
            "tokens_per_s": round(wl.T / (head_summary["fused_ms"] * 1e-3), 1),
            "unfused_ms_per_step_median": round(head_summary["unfused_ms"], 4),
            "speedup_vs_unfused": round(head_summary["unfused_ms"] / head_summary["fused_ms"], 3),
            **head_orders},
    }
    del r
    # (the default set of workloads only) the DeepSeek-shaped workloads again
    # with FP8 weights, each right after its bf16 run while the weights it
    # quantises are still on the device
    fp8_names = ([] if args.no_fp8 or args.others is not None or args.weights == "fp8"
                 or args.backward or args.reroute
                 else [n for n in FP8_WORKLOADS if n == args.workload or n in others])
    fp8_out = {}

    def run_fp8(name):
        log(f"{name} with FP8 weights")
        rf = run_workload(args, make(name), weights, dev, headline=False, fp8=True)
        fp8_out[name] = {"weights": "e4m3 codes, power-of-two fp32 scale per 128 x 128 block",
                         **summary_of(args, rf)}
    if args.workload in fp8_names:
        run_fp8(args.workload)
    others_out = {}
    for name in others:
        wo = make(name)
        ro = run_workload(args, wo, weights, dev, headline=False)
        others_out[name] = summary_of(args, ro)
        del ro
        if name in fp8_names:
            run_fp8(name)
    line["others"] = others_out or None
    line["fp8_weights"] = fp8_out or None
    if args.arrivals > 0:
        log(f"arrivals: {args.arrivals} source batches of {args.workload}")
        line["arrivals"] = arrivals_bench(args, args.workload, weights, dev)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

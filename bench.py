#!/usr/bin/env python3
"""Benchmark of the MoE expert path on one MI355X.

One step = one whole MoE layer on one batch: router logits -> top-k routing ->
dispatch (plan + permutation) -> grouped GEMM1 + SwiGLU -> grouped GEMM2 ->
weighted combine, all through the library's C ABI on one HIP stream, inputs
resident in HBM.  Default workload: the Mixtral-shaped bf16 prefill layer
(T=4096 tokens, d_model=4096, d_ff=14336, 8 experts, top-2), synthetic seeded
inputs.  Prints ONE JSON line.

Also reports, for the dominant kernel (GEMM1 + SwiGLU), its achieved MFMA
throughput against the bf16 dense peak, and the CPU oracle timed on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
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
STEPS = ("router", "route", "dispatch", "ffn_up", "ffn_down", "combine")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="mixtral_prefill")
    p.add_argument("--reroute", action="store_true",
                   help="route with capacity-overflow rerouting (moe_route_reroute)")
    p.add_argument("--weights", choices=("native", "fp8"), default="native",
                   help="fp8: quantise the packed bf16 expert weights to E4M3 codes with "
                        "128 x 128 block scales (moe_quantize_fp8, untimed) and run the FFN "
                        "steps on them")
    p.add_argument("--backward", action="store_true",
                   help="also time a training step: the forward with the SwiGLU pre-activations "
                        "kept, then the whole backward pass (gradients of x, the gate logits "
                        "or router, and the expert weights); reported under 'training'")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=256)
    p.add_argument("--traffic", default=None,
                   help="JSON file with counter-derived HBM bytes per launch of the dominant "
                        "kernel (default: profiles/traffic_<workload>.json if present)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (the counter calibration kernel)")
    p.add_argument("--traffic-from", default=None, metavar="DIR",
                   help="turn rocprofv3 --pmc databases under DIR/{fetch,write,copy_fetch,"
                        "copy_write} into profiles/traffic_<workload>.json and exit")
    p.add_argument("--counters-from", default=None, metavar="DIR",
                   help="summarise a rocprofv3 --pmc database under DIR taken with "
                        + " ".join(MFMA_COUNTERS) + " (MFMA busy fraction and counted "
                        "MFMA flops per kernel) and exit")
    return p.parse_args()


# ---- HBM traffic of the dominant kernel from hardware counters -------------
#
# FETCH_SIZE and WRITE_SIZE (KiB per dispatch, summed over the channels) are
# taken in two rocprofv3 --pmc passes over a short bench run, and in two passes
# over a plain device copy of known size; the copy's counted bytes over its
# true bytes is the scale applied to the kernel's counts.  The result records a
# hash of the kernel's sources: once they change, the stored traffic is stale
# and the bench reports null.

DOMINANT = "moe_ffn_up"                         # one GEMM1 + SwiGLU pass over all local rows
# the kernels that pass launches (demangled name prefixes): the pipelined
# 256-row / remainder kernels, the register-staged few-rows kernel, fp32
DOMINANT_KERNELS = ("gemm_bf16_pipe<true", "gemm_bf16_kernel<32, 128, 64, 1, 4, true",
                    "gemm_f32_kernel<true")
DOMINANT_SOURCES = ("routing_dispatch_expert_moe_amd/csrc/ffn_big.hip",
                    "routing_dispatch_expert_moe_amd/csrc/gemm_pipe.h",
                    "routing_dispatch_expert_moe_amd/csrc/ffn_bf16.hip",
                    "routing_dispatch_expert_moe_amd/csrc/tile_sched.h",
                    "routing_dispatch_expert_moe_amd/csrc/common.h")
COPY_BYTES = 1 << 30


def sources_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in DOMINANT_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


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
    """{dispatch_id: (kernel_name, value summed over dimensions)} from rocprofv3 databases."""
    import glob
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
    d = args.traffic_from
    res = {}
    for ctr, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        copy = [v for n, v in _pmc_per_dispatch(os.path.join(d, "copy_" + sub), ctr).values()
                if "copy" in n.lower() or "elementwise" in n.lower()]
        kern = [v for n, v in _pmc_per_dispatch(os.path.join(d, sub), ctr).values()
                if any(p in n for p in DOMINANT_KERNELS)]
        if not copy or not kern:
            raise SystemExit(f"{ctr}: found {len(copy)} copy and {len(kern)} kernel dispatches")
        copy_kib = float(np.median(copy))
        scale = (COPY_BYTES / 1024.0) / copy_kib   # true KiB per counted KiB
        res[ctr] = {"copy_counted_kib": copy_kib, "scale": scale,
                    "kernel_dispatches": len(kern),
                    "kernel_counted_kib_per_dispatch": float(np.mean(kern))}
    # the dominant pass launches len(DOMINANT_KERNELS)-many kernels per call at most;
    # bytes per call = sum over its kernels of their mean counted KiB, scaled
    per_call = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        groups = {}
        sub = "fetch" if ctr == "FETCH_SIZE" else "write"
        for n, v in _pmc_per_dispatch(os.path.join(d, sub), ctr).values():
            if any(p in n for p in DOMINANT_KERNELS):
                groups.setdefault(n.split("(")[0], []).append(v)
        per_call[ctr] = sum(float(np.mean(v)) for v in groups.values()) * 1024.0 * res[ctr]["scale"]
        res[ctr]["kernels"] = {k: float(np.mean(v)) for k, v in groups.items()}
    out = {DOMINANT: {"fetch_bytes": per_call["FETCH_SIZE"], "write_bytes": per_call["WRITE_SIZE"],
                      "bytes": per_call["FETCH_SIZE"] + per_call["WRITE_SIZE"]},
           "workload": args.workload, "sources_sha256_16": sources_hash(), "counters": res}
    path = args.traffic or os.path.join(ROOT, "profiles", f"traffic_{args.workload}.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out[DOMINANT]))


def load_traffic(args):
    if getattr(args, "weights", "native") != "native":
        return None, "counters were taken with the native-precision weights"
    path = args.traffic or os.path.join(ROOT, "profiles", f"traffic_{args.workload}.json")
    if not os.path.exists(path):
        return None, "no counter file"
    with open(path) as fh:
        t = json.load(fh)
    if t.get("workload") != args.workload:
        return None, "counter file is for another workload"
    if t.get("sources_sha256_16") != sources_hash():
        return None, "kernel sources changed since the counters were taken"
    return t[DOMINANT]["bytes"], "rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a 1 GiB copy"


def smi_snapshot():
    """Graphics and memory clocks and socket power read from the driver's sysfs
    files (plain reads; no program is started): {"sclk_mhz", "mclk_mhz",
    "socket_power_w", "power_cap_w"}, or None where they are missing."""
    import glob
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
    codes; their block scales add 4 B per 128 x 128 block)."""
    b = 2 if wl.dtype == "bf16" else 4
    if wb is None:
        wb = b
    T, d, f, E, k = wl.T, wl.d, wl.f, wl.E, wl.k
    m = {
        "router": (2.0 * T * d * E if wl.w_gate is not None else 0.0,
                   (T * d * b + d * E * 4 + T * E * 4) if wl.w_gate is not None else 0.0),
        "route": (0.0, T * E * 4 + T * k * 8),
        "dispatch": (0.0, 12.0 * T * k + T_read * d * b + n * d * b),
        "ffn_up": (4.0 * n * d * f, touched * 2.0 * f * d * wb + n * d * b + n * f * b),
        "ffn_down": (2.0 * n * f * d, touched * 1.0 * d * f * wb + n * f * b + n * d * b),
        "combine": (0.0, n * d * b + T * k * 8 + T * d * b),
    }
    return m


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
    fl = sum(v[0] for v in model.values() if v is not None) - model["ffn_up"][0]
    # the dominant backward call: the longest one
    dom = max(TRAIN_STEPS[6:], key=lambda k: per[k]["ms"])
    dfl, dby = model[dom]
    dms = per[dom]["ms"]
    if dfl / (PEAK_BF16_TFLOPS * 1e12) >= dby / (PEAK_HBM_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": round(dfl / (dms * 1e-3) / 1e12, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(dby / (dms * 1e-3) / 1e9, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof.update(call=dom, frac=round(roof["achieved"] / roof["peak"], 4), avg_launch_ms=dms,
                algorithmic_flops_per_launch=dfl, algorithmic_bytes_per_launch=dby)
    return {"ms_per_step": round(ms_step, 4), "tokens_per_s": round(wl.T / (ms_step * 1e-3), 1),
            "backward_ms": round(bwd_ms, 4), "step_tflops": round(fl / (ms_step * 1e-3) / 1e12, 2),
            "per_call": per, "roofline": roof,
            "note": "one step = forward (pre-activations kept) + backward: combine, gate and "
                    "router backward, dh and SwiGLU', dx, fp32 weight gradients; HIP events "
                    "around every call on the launch stream"}


def main():
    args = parse()
    if args.traffic_from:
        traffic_from(args)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.counters_from:
        counters_from(args)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; "
                                   f"--gpus {args.gpus} is not supported (the path is single-GPU)"}))
        sys.exit(2)
    import torch
    import routing_dispatch_expert_moe_amd as M
    from workloads import make

    dev = torch.device("cuda:0")
    wl = make(args.workload)
    log(f"workload {wl.name}: T={wl.T} d={wl.d} f={wl.f} E={wl.E} k={wl.k} dtype={wl.dtype}")

    # weights: generated on the host, uploaded, packed once (untimed)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    w13 = torch.empty((wl.E_loc, 2 * wl.f, wl.d), dtype=tdt, device=dev)
    w2p = torch.empty((wl.E_loc, wl.d, wl.f), dtype=tdt, device=dev)
    host_w = []
    keep_host = not args.no_cpu_baseline

    def up(a):
        return bf16_dev(a, dev) if wl.dtype == "bf16" else torch.from_numpy(a).to(dev)

    train = args.backward
    if train:   # the backward operands: [W1 | W3] rows per d, and W2 as it is
        w13_t = torch.empty((wl.E_loc, wl.d, 2 * wl.f), dtype=tdt, device=dev)
        w2_t = torch.empty((wl.E_loc, wl.f, wl.d), dtype=tdt, device=dev)
    for c0 in range(0, wl.E_loc, 8):
        ids = list(range(wl.e_begin + c0, wl.e_begin + min(wl.E_loc, c0 + 8)))
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
    log("weights packed")

    C = M.moe_capacity(wl.T, wl.k, wl.E, wl.capacity_factor)
    fp8 = args.weights == "fp8"
    if fp8:
        if wl.dtype != "bf16":
            raise SystemExit("--weights fp8 needs a bf16 workload")
        q13, s13 = M.moe_quantize_fp8(w13)
        q2, s2 = M.moe_quantize_fp8(w2p)
        torch.cuda.synchronize()
        del w13, w2p
        torch.cuda.empty_cache()
        w13, w2p = q13, q2
        log("weights quantised to E4M3 with 128 x 128 block scales")
    layer = M.MoELayer(w13, w2p, E=wl.E, k=wl.k, gate=wl.gate, T=wl.T, capacity=C,
                       w13_scale=s13 if fp8 else None, w2_scale=s2 if fp8 else None,
                       reroute=args.reroute,
                       e_begin=wl.e_begin, e_end=wl.e_end)
    x = up(wl.x)
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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    status = M.moe_check_error(layer.ws)
    if status != 0:
        raise RuntimeError(f"device error {status}")
    n = int(layer.plan.n_kept[0].item())
    counts = layer.plan.counts.cpu().numpy()[wl.e_begin:wl.e_end]
    touched = int((np.minimum(counts, C if C >= 0 else counts.max()) > 0).sum())
    pp = layer.plan.pair_pos.cpu().numpy()[:wl.T * wl.k].reshape(wl.T, wl.k)
    T_read = int((pp >= 0).any(axis=1).sum())
    log(f"n_kept={n} experts touched={touched} counts min={counts.min()} max={counts.max()}")

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    smi_before = smi_snapshot()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    smi_after = smi_snapshot()
    ms_step = (t1 - t0) * 1e3 / args.steps

    # the same steps with the 256 MB Infinity Cache (MALL) evicted before each:
    # a 1 GiB write between steps, outside the events, so that no step starts
    # with its inputs or weights cache-resident (per-step HIP-event times)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cev = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    for s in range(args.steps):
        scratch.fill_(s & 0xFF)
        step(cev[s])
    torch.cuda.synchronize()
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
    del scratch, src, dst
    cold_ms = {name: float(np.median([cev[s][i].elapsed_time(cev[s][i + 1])
                                      for s in range(args.steps)]))
               for i, name in enumerate(STEPS)}
    cold_step = float(np.median([cev[s][0].elapsed_time(cev[s][6]) for s in range(args.steps)]))

    # the same layer as one fused persistent launch (router logits stay a separate call)
    fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]

    def fused_step(ev=None):
        if ev is not None:
            ev[0].record()
        lg = layer.router(x, wg) if wg is not None else logits
        layer.forward_fused(x, lg)
        if ev is not None:
            ev[1].record()

    fused_ms = None
    if not fp8:   # the fused launch: bf16 / fp32 weights (with the layer's routing)
        for _ in range(args.warmup):
            fused_step()
        torch.cuda.synchronize()
        for s in range(args.steps):
            fused_step(fev[s])
        torch.cuda.synchronize()
        if M.moe_check_error(layer.ws) != 0:
            raise RuntimeError("device error in the fused layer")
        fused_ms = float(np.median([e[0].elapsed_time(e[1]) for e in fev]))
    unfused_ms = float(np.median([events[s][0].elapsed_time(events[s][6]) for s in range(args.steps)]))

    per = {}
    model = work_model(wl, n, touched, T_read, wb=(1 + 4.0 / (128 * 128)) if fp8 else None)
    cold = {name: {"ms": round(ms, 5),
                   "gbs": round(model[name][1] / (ms * 1e-3) / 1e9, 1) if model[name][1] else None}
            for name, ms in cold_ms.items()}
    for i, name in enumerate(STEPS):
        ms = float(np.mean([events[s][i].elapsed_time(events[s][i + 1]) for s in range(args.steps)]))
        fl, by = model[name]
        per[name] = {"ms": round(ms, 5),
                     "tflops": round(fl / (ms * 1e-3) / 1e12, 2) if fl else None,
                     "gbs": round(by / (ms * 1e-3) / 1e9, 1) if by else None}
    flops = sum(v[0] for v in model.values())
    bytes_ = sum(v[1] for v in model.values())
    tflops = flops / (ms_step * 1e-3) / 1e12
    gbs = bytes_ / (ms_step * 1e-3) / 1e9

    dom = "ffn_up"
    dom_ms = per[dom]["ms"]
    dom_fl, dom_by = model[dom]
    traffic, traffic_note = load_traffic(args)
    # the pass is bound by whichever of its algorithmic flops and bytes takes
    # longer at peak: MFMA with many rows per expert, HBM (weight streaming)
    # with few
    if dom_fl / (PEAK_BF16_TFLOPS * 1e12) >= dom_by / (PEAK_HBM_GBS * 1e9):
        bound, achieved, peak, unit = ("mfma", dom_fl / (dom_ms * 1e-3) / 1e12,
                                       PEAK_BF16_TFLOPS, "TFLOP/s")
    else:
        bound, achieved, peak, unit = ("hbm", dom_by / (dom_ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s")
    if wl.dtype != "bf16":
        kernel = f"{DOMINANT}: gemm_f32_kernel<SwiGLU>"
    elif layer.plan.max_rows // wl.E_loc <= 48:   # the launcher's few-rows rule
        kernel = (f"{DOMINANT}: gemm_bf16_kernel<SwiGLU{', FP8 weights' if fp8 else ''}>, "
                  "32-row tiles over every row")
    elif fp8:
        kernel = f"{DOMINANT}: gemm_bf16_kernel<SwiGLU, FP8 weights>, 64-row tiles"
    else:
        kernel = f"{DOMINANT}: gemm_bf16_pipe<SwiGLU>, 256-row tiles (+ remainder tiles)"
    roofline = {"bound": bound, "kernel": kernel,
                "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4),
                "traffic": round(traffic) if traffic is not None else None,
                "traffic_note": traffic_note,
                "algorithmic_flops_per_launch": dom_fl,
                "algorithmic_bytes_per_launch": dom_by, "avg_launch_ms": dom_ms}

    training = None
    if train:
        if fp8 or args.reroute:
            raise SystemExit("--backward takes native weights and plain top-k routing")
        training = train_bench(args, wl, layer, x, logits, wg, w13_t, w2_t, n, touched, T_read, dev)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle on {args.cpu_sample_tokens} tokens")
        rate, dt, n_tok, passes = cpu_baseline(wl, host_w, args.cpu_sample_tokens)
        cpu = {"value": round(rate, 2), "unit": "tokens/s", "cores": _CORES, "kind": "oracle",
               "sample": f"first {n_tok} of {wl.T} tokens of {wl.name} (capacity rule applied "
                         f"to the sample), whole layer in float64 (router..combine), "
                         f"{passes} pass(es), {dt:.1f} s timed"}

    line = {
        "metric": METRIC, "value": round(wl.T / (ms_step * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": wl.name, "tokens": wl.T, "d_model": wl.d, "d_ff": wl.f,
                   "experts": wl.E, "local_experts": wl.E_loc, "top_k": wl.k, "gate": wl.gate,
                   "capacity": C, "parallelism": "single GPU",
                   "weights": "e4m3 codes, fp32 scale per 128x128 block" if fp8 else wl.dtype,
                   "routing": "top-k with overflow rerouting" if args.reroute else "top-k"},
        "layer_tflops": round(tflops, 2), "layer_mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "layer_hbm_gbs": round(gbs, 1), "layer_hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "per_step": per, "roofline": roofline, "cpu_baseline": cpu,
        "mall_flushed": {"ms_per_step_median": round(cold_step, 4),
                         "per_step_median": cold,
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
        "fused": None if fused_ms is None else {
            "entry": "moe_forward_fused_reroute" if args.reroute else "moe_forward_fused",
            "ms_per_step_median": round(fused_ms, 4),
            "tokens_per_s": round(wl.T / (fused_ms * 1e-3), 1),
            "unfused_ms_per_step_median": round(unfused_ms, 4),
            "speedup_vs_unfused": round(unfused_ms / fused_ms, 3)},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

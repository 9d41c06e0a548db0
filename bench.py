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
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=256)
    p.add_argument("--traffic", default=None,
                   help="JSON file with counter-derived HBM bytes per launch of the dominant kernel")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def bf16_dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def work_model(wl, n, touched, T_read):
    """Algorithmic flops and HBM bytes per launch of each step."""
    b = 2 if wl.dtype == "bf16" else 4
    T, d, f, E, k = wl.T, wl.d, wl.f, wl.E, wl.k
    m = {
        "router": (2.0 * T * d * E if wl.w_gate is not None else 0.0,
                   (T * d * b + d * E * 4 + T * E * 4) if wl.w_gate is not None else 0.0),
        "route": (0.0, T * E * 4 + T * k * 8),
        "dispatch": (0.0, 12.0 * T * k + T_read * d * b + n * d * b),
        "ffn_up": (4.0 * n * d * f, touched * 2.0 * f * d * b + n * d * b + n * f * b),
        "ffn_down": (2.0 * n * f * d, touched * 1.0 * d * f * b + n * f * b + n * d * b),
        "combine": (0.0, n * d * b + T * k * 8 + T * d * b),
    }
    return m


def cpu_baseline(wl, host_w, n_tok):
    """The CPU oracle (float64) on the first n_tok tokens of the workload."""
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


def main():
    args = parse()
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

    for c0 in range(0, wl.E_loc, 8):
        ids = list(range(wl.e_begin + c0, wl.e_begin + min(wl.E_loc, c0 + 8)))
        a, b, c = wl.stacked_weights(ids)
        if keep_host:
            host_w.extend(zip(a, b, c))
        M.moe_pack_weights(up(a), up(b), up(c), w13[c0:c0 + len(ids)], w2p[c0:c0 + len(ids)])
    torch.cuda.synchronize()
    log("weights packed")

    C = M.moe_capacity(wl.T, wl.k, wl.E, wl.capacity_factor)
    layer = M.MoELayer(w13, w2p, E=wl.E, k=wl.k, gate=wl.gate, T=wl.T, capacity=C,
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
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps

    per = {}
    model = work_model(wl, n, touched, T_read)
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
    dom_fl = model[dom][0]
    achieved = dom_fl / (dom_ms * 1e-3) / 1e12
    traffic = None
    if args.traffic and os.path.exists(args.traffic):
        with open(args.traffic) as fh:
            traffic = json.load(fh).get(dom)
    roofline = {"bound": "mfma", "kernel": "gemm_bf16_kernel<SwiGLU> (moe_ffn_up)",
                "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "algorithmic_flops_per_launch": dom_fl, "avg_launch_ms": dom_ms}

    cpu = None
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle on {args.cpu_sample_tokens} tokens")
        rate, dt = cpu_baseline(wl, host_w, args.cpu_sample_tokens)
        cpu = {"value": round(rate, 2), "unit": "tokens/s", "cores": _CORES, "kind": "oracle",
               "sample": f"first {args.cpu_sample_tokens} of {wl.T} tokens of {wl.name}, whole "
                         f"layer in float64 (router..combine), {dt:.1f} s"}

    line = {
        "metric": METRIC, "value": round(wl.T / (ms_step * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": wl.name, "tokens": wl.T, "d_model": wl.d, "d_ff": wl.f,
                   "experts": wl.E, "local_experts": wl.E_loc, "top_k": wl.k, "gate": wl.gate,
                   "capacity": C, "parallelism": "single GPU"},
        "layer_tflops": round(tflops, 2), "layer_mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "layer_hbm_gbs": round(gbs, 1), "layer_hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "per_step": per, "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

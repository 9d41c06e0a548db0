"""Host-side logic of bench.py (no GPU): the counter summaries read from
rocprofv3 databases, the stored-traffic bookkeeping, and the single-GPU rule.
The databases are small synthetic sqlite files with the counter table the
summaries read (one row per dispatch and counter)."""
import contextlib
import csv
import io
import json
import os
import sqlite3
import subprocess
import sys
from types import SimpleNamespace

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

GEMM = "void moe::gemm_bf16_pipe<true, 256, 256, 4, 0, false>(unsigned short const*, int const*)"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::copy_kernel>(int)"


def write_db(path, rows):
    """rows: (dispatch_id, kernel_name, counter_name, value)."""
    os.makedirs(os.path.dirname(path), exist_ok=True)
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (dispatch_id integer, kernel_name text, "
                "counter_name text, value real)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def run_quiet(fn, *a):
    out = io.StringIO()
    with contextlib.redirect_stdout(out):
        fn(*a)
    return out.getvalue()


def test_counters_summary(tmp_path):
    # two dispatches of one GEMM: 3000 active cycles per XCD, pipes busy 40 %
    # of them, 1e6 MFMA ops of 512 flops; a kernel without MFMA work is left out
    cycles = 3000
    busy = 0.4 * cycles * bench.N_SIMD
    rows = []
    for did in (1, 2):
        rows += [(did, GEMM, "GRBM_GUI_ACTIVE", cycles * bench.N_XCD),
                 (did, GEMM, "SQ_VALU_MFMA_BUSY_CYCLES", busy / 2),   # two rows: summed
                 (did, GEMM, "SQ_VALU_MFMA_BUSY_CYCLES", busy / 2),
                 (did, GEMM, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e6),
                 (did, GEMM, "SQ_LDS_BANK_CONFLICT", 7.0)]
    rows += [(3, COPY, "GRBM_GUI_ACTIVE", 800.0), (3, COPY, "SQ_VALU_MFMA_BUSY_CYCLES", 0.0)]
    write_db(str(tmp_path / "pmc" / "a_results.db"), rows)
    out = run_quiet(bench.counters_from, SimpleNamespace(counters_from=str(tmp_path / "pmc")))
    recs = [json.loads(line) for line in out.splitlines()]
    assert len(recs) == 1
    r = recs[0]
    assert r["kernel"] == GEMM.split("(")[0] and r["dispatches"] == 2
    assert r["active_cycles"] == cycles
    assert r["mfma_busy_frac"] == pytest.approx(0.4)
    assert r["mfma_flops_counted"] == pytest.approx(512e6)
    assert r["lds_bank_conflict_cycles"] == pytest.approx(7.0)


def test_traffic_from_scales_by_the_copy(tmp_path, monkeypatch):
    # the copy's counters read 2x its true bytes, so the kernels' counts halve;
    # each pass's bytes per call add up its kernels (two for a split GEMM1)
    copy_kib = 2.0 * bench.COPY_BYTES / 1024
    tail = GEMM.replace("256, 256, 4, 0", "128, 256, 6, 4")
    comb = "void moe::combine_kernel<true>(unsigned short const*)"
    d = tmp_path / "tr"
    for ctr, sub, kib in (("FETCH_SIZE", "fetch", 4096.0), ("WRITE_SIZE", "write", 1024.0)):
        write_db(str(d / sub / "k_results.db"),
                 [(1, GEMM, ctr, kib), (2, GEMM, ctr, kib), (3, tail, ctr, 10.0),
                  (4, comb, ctr, 6.0), (5, COPY, ctr, 5.0)])
        write_db(str(d / ("copy_" + sub) / "c_results.db"),
                 [(1, COPY, ctr, copy_kib), (2, COPY, ctr, copy_kib)])
    args = SimpleNamespace(traffic_from=str(d), profiles_dir=str(tmp_path), workload="mixtral_prefill")
    run_quiet(bench.traffic_from, args)
    dst = tmp_path / "traffic_mixtral_prefill.json"
    t = json.loads(dst.read_text())
    up = t["passes"][bench.DOMINANT]
    assert up["fetch_bytes"] == pytest.approx((4096.0 + 10.0) * 1024 / 2)
    assert up["write_bytes"] == pytest.approx((1024.0 + 10.0) * 1024 / 2)
    assert up["bytes"] == pytest.approx(up["fetch_bytes"] + up["write_bytes"])
    assert t["passes"]["combine"]["bytes"] == pytest.approx(2 * 6.0 * 1024 / 2)
    assert "ffn_down" not in t["passes"]
    assert t["sources_sha256_16"] == bench.sources_hash()

    # the stored figure is used while the sources are unchanged, else dropped
    load_args = SimpleNamespace(weights="native", profiles_dir=str(tmp_path))
    val, note = bench.load_stored(load_args, "traffic", "mixtral_prefill")
    assert val["passes"][bench.DOMINANT]["bytes"] == pytest.approx(up["bytes"])
    assert bench.load_stored(load_args, "traffic", "dsv3_decode")[0] is None
    monkeypatch.setattr(bench, "sources_hash", lambda: "0" * 16)
    val, note = bench.load_stored(load_args, "traffic", "mixtral_prefill")
    assert val is None and "changed" in note
    fp8 = SimpleNamespace(weights="fp8", profiles_dir=str(tmp_path))
    assert bench.load_stored(fp8, "traffic", "mixtral_prefill")[0] is None


def test_trace_summary_takes_the_timed_steps(tmp_path):
    """warm-up steps, then timed steps, then cache-evicted steps: the summary
    averages the timed steps of each pass, its kernels added per step."""
    big = "void moe::gemm_bf16_pipe<true, 256, 256, 4, 3, false>(unsigned short const*)"
    tail = "void moe::gemm_bf16_pipe<true, 128, 256, 6, 4, false>(unsigned short const*)"
    comb = "void moe::combine_kernel<true>(unsigned short const*)"
    W, K = 2, 3
    rows, t = [], 1000
    for step in range(W + 2 * K):
        timed = W <= step < W + K
        for name, us in ((big, 100 + (10 * step if timed else 500)), (tail, 20), (comb, 5)):
            rows.append((t, t + int(us * 1000), name))
            t += int(us * 1000) + 50
    d = tmp_path / "kt" / "host" / "123"
    d.mkdir(parents=True)
    with open(d / "kt_kernel_trace.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for s0, s1, n in rows:
            w.writerow(["KERNEL_DISPATCH", n, s0, s1])
    (tmp_path / "kt" / "bench.json").write_text(json.dumps(
        {"per_step": {"ffn_up": {"ms": 0.141}, "combine": {"ms": 0.005}}}) + "\n")
    args = SimpleNamespace(trace_from=str(tmp_path / "kt"), profiles_dir=str(tmp_path),
                           workload="dsv3_prefill_zipf", steps=K, warmup=W)
    run_quiet(bench.trace_from, args)
    out = json.loads((tmp_path / "kernel_times_dsv3_prefill_zipf.json").read_text())
    up = out["passes"]["ffn_up"]
    assert up["launches_per_call"] == 2
    assert up["per_step_us"] == pytest.approx([100 + 20 + 10 * s for s in range(W, W + K)])
    assert up["mean_us"] == pytest.approx(120 + 10 * (W + 1))
    assert out["passes"]["combine"]["mean_us"] == pytest.approx(5)
    assert out["bench_event_mean_us"]["ffn_up"] == pytest.approx(141)
    md = (tmp_path / "kernels_dsv3_prefill_zipf.md").read_text()
    assert "gemm_bf16_pipe<true, 256, 256, 4, 3, false>" in md and "| ffn_up |" in md


def test_roofline_of_picks_the_longer_bound():
    # 2.5 TFLOP in 2 ms: MFMA bound 1 ms -> half the MFMA roofline
    r = bench.roofline_of(2.5e12, 1e9, 2.0)
    assert r["bound"] == "mfma" and r["frac"] == pytest.approx(0.5)
    assert r["achieved"] == pytest.approx(1250.0)
    # 16 GB in 4 ms: HBM bound 2 ms
    r = bench.roofline_of(1e12, 16e9, 4.0)
    assert r["bound"] == "hbm" and r["frac"] == pytest.approx(0.5) and r["achieved"] == 4000.0
    assert bench.pass_of("void moe::permute_rows_kernel(int)") == "permute"
    assert bench.pass_of("void moe::combine_backward_kernel<true>(int)") is None
    assert bench.pass_of("void moe::gemm_bf16_kernel<32, 128, 64, 1, 4, false, 0, false>(x)") == "ffn_down"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_arrivals_join_is_expert_major_then_source_order():
    """The rows a rank receives from several sources are joined expert by
    expert, each expert's rows in source order, with matching offsets; a
    source with no row for an expert adds nothing."""
    import torch
    d = 3
    # source 0: experts 0, 1, 2 hold 2, 0, 1 rows; source 1: 1, 2, 0 rows
    x0 = torch.tensor([[0., 0, 0], [0, 0, 1], [0, 2, 0]])
    x1 = torch.tensor([[1., 0, 0], [1, 1, 0], [1, 1, 1]])
    xp, off = bench.join_arrivals([(x0, [0, 2, 2, 3]), (x1, [0, 1, 3, 3])], 3)
    assert off == [0, 3, 5, 6]
    want = torch.stack([x0[0], x0[1], x1[0],      # expert 0: source 0, then source 1
                        x1[1], x1[2],             # expert 1: source 1 only
                        x0[2]])                   # expert 2: source 0 only
    assert torch.equal(xp, want) and xp.shape == (6, d)
    # no rows at all: one zero row keeps the buffer non-empty, offsets all zero
    xe, oe = bench.join_arrivals([(x0[:0], [0, 0]), (x1[:0], [0, 0])], 1)
    assert oe == [0, 0] and xe.shape == (1, d)

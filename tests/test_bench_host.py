"""Host-side logic of bench.py (no GPU): the counter summaries read from
rocprofv3 databases, the stored-traffic bookkeeping, and the single-GPU rule.
The databases are small synthetic sqlite files with the counter table the
summaries read (one row per dispatch and counter)."""
import contextlib
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
    # the copy's counters read 2x its true bytes, so the kernel's counts halve
    copy_kib = 2.0 * bench.COPY_BYTES / 1024
    d = tmp_path / "tr"
    for ctr, sub, kib in (("FETCH_SIZE", "fetch", 4096.0), ("WRITE_SIZE", "write", 1024.0)):
        write_db(str(d / sub / "k_results.db"),
                 [(1, GEMM, ctr, kib), (2, GEMM, ctr, kib), (3, COPY, ctr, 5.0)])
        write_db(str(d / ("copy_" + sub) / "c_results.db"),
                 [(1, COPY, ctr, copy_kib), (2, COPY, ctr, copy_kib)])
    dst = tmp_path / "traffic.json"
    args = SimpleNamespace(traffic_from=str(d), traffic=str(dst), workload="mixtral_prefill")
    run_quiet(bench.traffic_from, args)
    t = json.loads(dst.read_text())
    up = t[bench.DOMINANT]
    assert up["fetch_bytes"] == pytest.approx(4096.0 * 1024 / 2)
    assert up["write_bytes"] == pytest.approx(1024.0 * 1024 / 2)
    assert up["bytes"] == pytest.approx(up["fetch_bytes"] + up["write_bytes"])
    assert t["sources_sha256_16"] == bench.sources_hash()

    # the stored figure is used while the sources are unchanged, else dropped
    load_args = SimpleNamespace(weights="native", traffic=str(dst), workload="mixtral_prefill")
    val, note = bench.load_traffic(load_args)
    assert val == pytest.approx(up["bytes"]) and "FETCH_SIZE" in note
    assert bench.load_traffic(SimpleNamespace(weights="native", traffic=str(dst),
                                              workload="dsv3_decode"))[0] is None
    monkeypatch.setattr(bench, "sources_hash", lambda: "0" * 16)
    val, note = bench.load_traffic(load_args)
    assert val is None and "changed" in note
    assert bench.load_traffic(SimpleNamespace(weights="fp8", traffic=str(dst),
                                              workload="mixtral_prefill"))[0] is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]

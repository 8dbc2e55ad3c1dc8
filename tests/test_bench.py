"""bench.py on the CPU: its command-line contract, the digest guard on the
counter table, the profile summaries it prints, and the algorithmic flops
and bytes its metric divides by, checked against closed forms of the
workloads (effective work 2 * nnz * N; compulsory bytes = the packed operand,
the touched rows of B and C, each once)."""
import contextlib
import io
import json
import os
import sqlite3
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    sys.path.insert(0, ROOT)
    import bench
    return bench


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_traffic_is_reported_only_for_the_current_library(bench, tmp_path, monkeypatch):
    dig = bench.library_digest()
    table = tmp_path / "hbm_traffic.md"
    table.write_text(
        "| workload | kernel | library digest | FETCH_SIZE KiB | WRITE_SIZE KiB | factors | bytes per launch |\n"
        "|---|---|---|---|---|---|---|\n"
        f"| w_now | k1 | {dig} | 1.0 | 2.0 | 2.3333, 1.0000 | 123456 |\n"
        "| w_old | k1 | 0123456789abcdef | 1.0 | 2.0 | 2.3333, 1.0000 | 999 |\n")
    monkeypatch.setattr(bench, "TRAFFIC_TABLE", str(table))
    assert bench.measured_traffic("w_now", "k1") == 123456
    assert bench.measured_traffic("w_now", "k2") is None       # another kernel
    assert bench.measured_traffic("w_old", "k1") is None       # counters of another build
    assert bench.measured_traffic("w_none", "k1") is None


def test_roofline_picks_the_longer_bound(bench, monkeypatch):
    monkeypatch.setattr(bench, "measured_traffic", lambda w, k: None)

    class W:
        name = "x"
    # 1 GB and 1 TFLOP in 1 ms: HBM at 8 TB/s needs 0.125 ms, bf16 MFMA 0.4 ms
    bind, other = bench.roofline(W, "k", 1e12, 1e9, "bf16", 1.0)
    assert bind["bound"] == "mfma" and bind["frac"] == pytest.approx(1000 / 2500, abs=1e-4)
    assert other["bound"] == "hbm" and other["frac"] == pytest.approx(1000 / 8000, abs=1e-4)
    bind, other = bench.roofline(W, "k", 1e9, 1e10, "i8", 2.0)
    assert bind["bound"] == "hbm" and bind["achieved"] == pytest.approx(5000.0)
    bind, other = bench.roofline(W, "k", 1e9, 1e9, "f32", 1.0)
    assert bind["bound"] == "hbm" and other is None


def _stdout(fn, *a):
    buf = io.StringIO()
    with contextlib.redirect_stdout(buf):
        fn(*a)
    return buf.getvalue()


def test_trace_and_counter_summaries(bench, tmp_path):
    d = tmp_path / "trace" / "box"
    d.mkdir(parents=True)
    con = sqlite3.connect(str(d / "run_results.db"))
    con.execute("create table kernels (name text, duration integer)")
    name = "void sdm::(anonymous namespace)::bcsr_bf16_pair<256, 128, 3>(int4 const*)"
    con.executemany("insert into kernels values (?, ?)",
                    [(name, 1000), (name, 3000), (name, 2000), ("copy_kernel", 500)])
    con.commit()
    con.close()
    out = _stdout(bench.trace_summary, str(tmp_path / "trace"))
    row = next(line for line in out.splitlines() if line.startswith("| bcsr_bf16_pair |"))
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[1] == "3" and float(cells[2]) == 2.0 and float(cells[3]) == 2.0  # calls, avg, median (us)
    assert float(cells[4]) == 1.0 and float(cells[5]) == 3.0
    c = tmp_path / "pmc" / "x"
    c.mkdir(parents=True)
    (c / "p_counter_collection.csv").write_text(
        "Kernel_Name,Counter_Name,Counter_Value\n"
        f"\"{name}\",FETCH_SIZE,100\n\"{name}\",FETCH_SIZE,300\nother,FETCH_SIZE,7\n")
    out = _stdout(bench.pmc_summary, str(tmp_path / "pmc"))
    line = next(l for l in out.splitlines() if l.startswith("bcsr_bf16_pair"))
    assert "dispatches=   2" in line and "mean=200" in line


def _setup_host(w):
    """The parts of bench.setup that run on the host: inputs and packing."""
    import sparse_dense_matrix_amd as S
    import synth
    a = synth.make_a(w)
    if w.fmt == "bcsr":
        M = S.spmm_pack_bcsr(a["dense"], w.block, w.block)
    else:
        M = S.spmm_pack_24(a["dense"])
    return {"a": a, "M": M, "info": S.spmm_matrix_info(M)}


@pytest.mark.parametrize("name, nnzb, kb", [("bcsr_4096_b64_90", 410, 64),
                                            ("bcsr_prefill_18944x3584", 1658, 56)])
def test_bcsr_work_and_bytes(bench, name, nnzb, kb):
    import synth
    w = synth.WORKLOADS[name]
    d = _setup_host(w)
    flops, nbytes, dtype = bench.algorithmic(w, d)
    assert dtype == "bf16" and d["info"]["nnzb"] == nnzb
    assert flops == 2.0 * nnzb * 64 * 64 * w.n
    # block columns a uniform 10% mask leaves untouched, counted from the generator's ids
    ids = synth.make_a(w)["block_ids"]
    touched = len(np.unique(np.asarray(ids) % kb))
    a_bytes = nnzb * 64 * 64 * 2 + 4 * (w.m // 64 + 1) + 4 * nnzb
    assert nbytes == a_bytes + touched * 64 * w.n * 2 + w.m * w.n * 2


def test_24_work_and_bytes(bench):
    import synth
    w = synth.WORKLOADS["sp24_i8_8192"]
    d = _setup_host(w)
    flops, nbytes, dtype = bench.algorithmic(w, d)
    assert dtype == "i8"
    assert flops == 2.0 * (8192 * 8192 // 2) * 2048          # 137.4 GOP
    # compressed values, 2-bit positions, B and int32 C once: 125.8 MB
    assert nbytes == 8192 * 4096 + 8192 * 8192 // 8 + 8192 * 2048 + 8192 * 2048 * 4

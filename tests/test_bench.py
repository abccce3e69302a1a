"""Host-side logic of bench.py (CPU): the algorithmic byte counts behind every
reported GB/s and roofline fraction, the guard that keeps stale counter
traffic out of the JSON line, the single-GPU refusal and the CPU-baseline
record."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_per_token():
    # single pass: the sources read once, out written once (fwd); sources and
    # dout read once, dsources written once (bwd); 8N bytes of saved rstd/alpha
    N, D = 9, 7168
    fwd, bwd, fe, be = bench.algo_bytes(1, N, D)
    assert fwd == 2 * N * D + 2 * D + 8 * N == 143_432
    assert bwd == 4 * N * D + 2 * D + 8 * N == 272_456
    assert fe == 4 * D  # w
    assert be == 4 * D + 8 * 1 * D + 4 * D  # w, one dw partial row written and read, dw


def test_algorithmic_bytes_of_the_default_workload():
    wl = synth.workload(1)
    fwd, bwd, fe, be = bench.algo_bytes(wl.T, wl.N, wl.D)
    assert (wl.T, wl.N, wl.D) == (4096, 9, 7168)
    # one attnres_bwd call: per-token bytes, w, 256 dw partial rows written and read, dw
    assert bwd + be == 1_130_717_184
    assert fwd + fe == 587_526_144
    # the committed counter record refers to the same byte count
    rec = json.load(open(bench.TRAFFIC_FILE))
    assert rec["algorithmic_bytes_per_call"] == bwd + be
    assert rec["fwd_kernel"]["algorithmic_bytes"] == fwd + fe


def test_partial_rows_follow_min_T_256():
    D = 64
    for T, P in [(1, 1), (100, 100), (256, 256), (257, 256), (100000, 256)]:
        _, _, _, be = bench.algo_bytes(T, 3, D)
        assert be == 8 * D + 8 * P * D


def test_kernel_hash_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    code = "__global__ void k(int* p) {\n  p[0] = 1;  // store\n}\n"
    a = tmp_path / "a.hip"
    a.write_text(code)
    monkeypatch.setattr(bench, "KERNEL_SRC", str(a))
    h0 = bench.kernel_source_hash()
    a.write_text("/* header\n comment */\n" + code.replace("// store", "// a different comment") + "\n\n")
    assert bench.kernel_source_hash() == h0
    a.write_text(code.replace("p[0] = 1", "p[0] = 2"))
    assert bench.kernel_source_hash() != h0


def test_stale_traffic_is_not_reported(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("__global__ void k() {}\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    rec = {"kernel_source_sha256_16": bench.kernel_source_hash(), "T": 4096, "N": 9, "D": 7168,
           "bytes_per_call": 123}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.load_traffic(4096, 9, 7168)["bytes_per_call"] == 123
    assert bench.load_traffic(4096, 9, 1024) is None  # another workload
    src.write_text("__global__ void k() { return; }\n")  # the kernel changed since the counters
    assert bench.load_traffic(4096, 9, 7168) is None
    f.write_text("not json")
    assert bench.load_traffic(4096, 9, 7168) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_record():
    wl = synth.Workload("bench_tiny", T=8, N=3, D=64)
    rec, ref = bench.cpu_baseline(wl, min_seconds=0.05)
    assert set(ref) == {"out", "rstd", "alpha", "dsrc", "dw"} and ref["dsrc"].shape == (3, 8, 64)
    assert rec["kind"] == "oracle" and rec["unit"] == "tokens/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert "fp64" in rec["sample"] and "8 tokens" in rec["sample"]


def test_parity_report_against_the_oracle_outputs():
    """The bench's parity record: the oracle's own values rounded to the device
    dtypes give rounding-level errors within the bars; a planted 5% error in dw
    is reported as such and fails them."""
    import numpy as np
    import torch

    wl = synth.Workload("bench_tiny", T=8, N=3, D=64)
    _, ref = bench.cpu_baseline(wl, min_seconds=0.0)
    as_dev = dict(out=torch.from_numpy(ref["out"]).to(torch.bfloat16), rstd=torch.from_numpy(ref["rstd"]).float(),
                  alpha=torch.from_numpy(ref["alpha"]).float(), dsrc=torch.from_numpy(ref["dsrc"]).to(torch.bfloat16),
                  dw=torch.from_numpy(ref["dw"]).float())
    e = bench.parity_report(torch, ref, **as_dev)
    assert e["within_bars"] and e["out_rel_l2"] < 4e-3 and e["dw_rel_l2"] < 1e-6
    bad = dict(as_dev, dw=as_dev["dw"] * 1.05)
    e = bench.parity_report(torch, ref, **bad)
    assert not e["within_bars"] and abs(e["dw_rel_l2"] - 0.05) < 1e-4
    assert np.isfinite(e["alpha_max_abs"])

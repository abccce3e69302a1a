"""Host-side logic of bench.py (CPU): the algorithmic byte counts behind every
reported GB/s and roofline fraction, the guard that keeps stale counter
traffic out of the JSON line, the single-GPU refusal, the oracle pass behind
the CPU-baseline and parity records, and the token sample."""
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
    assert be == 4 * D + 4 * D  # w read, dw written (the workspace's own traffic is reported apart)


def test_algorithmic_bytes_of_the_default_workload():
    wl = synth.workload(bench.DEFAULT_WORKLOAD)
    fwd, bwd, fe, be = bench.algo_bytes(wl.T, wl.N, wl.D)
    assert (wl.T, wl.N, wl.D) == (131072, 9, 7168) and wl.w_std == 0.5
    # one attnres_bwd call: per-token bytes, w, dw
    assert bwd + be == 131072 * 272_456 + 4 * 7168 + 4 * 7168 == 35_711_410_176
    assert fwd + fe == 131072 * 143_432 + 4 * 7168 == 18_799_947_776
    # a committed counter record, if present, refers to the same byte count
    f = bench.traffic_file(wl.T, wl.N, wl.D)
    assert os.path.basename(f) == "traffic_bwd_T131072_N9_D7168.json"
    if os.path.exists(f):
        rec = json.load(open(f))
        assert rec["algorithmic_bytes_per_call"] == bwd + be
        assert rec["fwd_kernel"]["algorithmic_bytes"] == fwd + fe


def test_workspace_traffic():
    """The backward's workspace traffic, reported next to (not inside) the
    algorithmic bytes: per-span partial rows and fold rows written and read,
    the exchange ring cleared (where the split backward runs); the one-token
    backward's partial rows otherwise."""
    D = 7168
    # T = 131072: 32768 spans of 4 tokens in 4 chunks, each folded into the 256
    # fold rows (written 4 times, re-read 3 times, read once by the final sum)
    assert bench.workspace_traffic(131072, 9, D) == 8 * 32768 * D + 4 * 256 * D * 8 + 4096 * 7 * 18 * 8
    # T = 100: 25 spans, one per fold row: no fold, the final sum reads the partial rows;
    # one slice per row (D = 64): no ring; two slices (D = 2048): the ring slots of 100 tokens cleared
    assert bench.workspace_traffic(100, 3, 64) == 8 * 25 * 64
    assert bench.workspace_traffic(100, 9, 2048) == 8 * 25 * 2048 + 100 * 2 * 18 * 8
    # N = 7 at D = 7168 takes the one-token backward: 256 partial rows
    assert bench.workspace_traffic(131072, 7, D) == 8 * 256 * D
    assert bench.workspace_traffic(5000, 9, 12288) == 8 * 256 * 12288
    assert bench.workspace_traffic(100, 9, 12288) == 8 * 100 * 12288


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
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    rec = {"kernel_source_sha256_16": bench.kernel_source_hash(), "T": 4096, "N": 9, "D": 7168,
           "bytes_per_call": 123}
    f = tmp_path / "traffic_bwd_T4096_N9_D7168.json"
    f.write_text(json.dumps(rec))
    assert bench.load_traffic(4096, 9, 7168)["bytes_per_call"] == 123
    assert bench.load_traffic(4096, 9, 1024) is None  # another workload: no record
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


def _rounded_outputs(wl, toks):
    """The oracle's own outputs rounded to the device dtypes: what an exact
    implementation would store."""
    import numpy as np
    import torch

    import oracle

    src, dout, w = wl.sources(), wl.dout(), wl.w()
    o_out, o_rstd, o_alpha = oracle.fwd(src, w, wl.eps)
    o_dsrc, o_dw = oracle.bwd(src, w, wl.eps, dout)
    bits = lambda a: torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    gpu = {"out_bits": bits(o_out), "rstd": o_rstd.astype(np.float32).astype(np.float64),
           "alpha": o_alpha.astype(np.float32).astype(np.float64),
           "dsrc_bits": bits(np.ascontiguousarray(o_dsrc[:, toks])), "dw": o_dw.astype(np.float32).astype(np.float64)}
    return (src, w, dout), gpu


def test_oracle_pass_record_and_parity():
    """The CPU-baseline record (fwd and bwd timed separately) and the parity
    record: the oracle's values rounded to the device dtypes are within the
    bars; a planted 5% error in dw, or one wrong token of out, is reported."""
    import torch

    wl = synth.Workload("bench_tiny", T=40, N=3, D=64)
    toks = bench.sample_tokens(wl.T)
    host, gpu = _rounded_outputs(wl, toks)
    rec, e = bench.oracle_pass(wl, host, gpu, toks, torch, chunk=16)
    assert rec["kind"] == "oracle" and rec["unit"] == "tokens/s" and rec["cores"] >= 1
    assert rec["value"] > 0 and rec["fwd_tokens_per_s"] > rec["value"] and rec["bwd_tokens_per_s"] > rec["value"]
    assert "40 tokens" in rec["sample"] and "fp64" in rec["sample"]
    assert e["within_bars"] and e["out_rel_l2"] < 4e-3 and e["dw_rel_l2"] < 1e-6, e
    bad = dict(gpu, dw=gpu["dw"] * 1.05)
    e = bench.oracle_pass(wl, host, bad, toks, torch, chunk=16)[1]
    assert not e["within_bars"] and abs(e["dw_rel_l2"] - 0.05) < 1e-4
    bad_out = gpu["out_bits"].copy()
    bad_out[17] = bad_out[3]  # one token's row replaced by another's
    e = bench.oracle_pass(wl, host, dict(gpu, out_bits=bad_out), toks, torch, chunk=16)[1]
    assert not e["within_bars"] and e["out_token_rel_l2"] > 0.1


def test_sample_tokens_cover_edges():
    toks = bench.sample_tokens(131072)
    assert {0, 1, 255, 256, 511, 131070, 131071} <= set(toks.tolist())
    assert len(toks) > 40 and toks.max() < 131072

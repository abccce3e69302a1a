#!/usr/bin/env python3
"""Benchmark: Attention Residuals forward + backward on one MI355X.

One step = attnres_fwd + attnres_bwd (every kernel of the operator) over one
batch of synthetic depth sources that are resident in HBM before timing
starts.  Default workload: T = 131072 local tokens, N = 9 sources, D = 7168,
w ~ N(0, 0.5) (peaked softmax) -- the 128K-token point where the pages quote
peak memory -- in bf16 storage with fp32 arithmetic.  Prints one JSON line
(N = 1 GPU):

  value         tokens/s over the K timed steps (whole job, one GPU)
  flushed       per-call medians with a 512 MiB cache flush before every call
  ceilings_GBps bandwidth the memory system gives to plain read / write /
                copy streams and to the operator's access patterns without
                arithmetic (libattnres_probes), measured on the same device
  roofline      the dominant call (attnres_bwd) against the 8 TB/s HBM peak,
                timed with HIP events on the stream the kernels run on
  cpu_baseline  the fp64 oracle on the host cores: fwd and bwd timed
                separately over the whole workload, and over a fixed token
                sample of every workload
  parity        the timed run's outputs against that oracle pass: out, alpha
                and rstd on every token, dsources on sampled tokens, dw over
                the whole batch

  block_batched_scores  one block's 24 sub-layer forwards the plain way vs
                one block-scores pass (MFMA) plus 24 forwards from its scores,
                and vs block scores + one block-sums pass (the shared sources'
                part of every sub-layer's weighted sum, fp32 or 24-bit
                elements) + 24 merged forwards

Flags: --gpus (1 only), --steps, --warmup, --workload (0..4, default 3),
--sweep (extra per-T / per-N lines with fwd and bwd timed separately and
caches flushed between reps), --no-cpu-baseline, --no-probes, --no-block,
--default-events (time with default HIP events instead of timing-only ones),
--decode / --block (only the decoding-size calls / only the block-batched
measurement, for profiles).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
PAGES_PEAK_GIB_128K = 35.03  # pages' fused figure at 128K local tokens (B300; context)
METRIC = "AttnRes fwd+bwd tokens/s and achieved HBM GB/s (% of peak), D=7168 N=9"
DEFAULT_WORKLOAD = 3
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "attention_residuals_depth_amd", "csrc", "attnres.hip")
PROBE_LIB = os.path.join(ROOT, "attention_residuals_depth_amd", "libattnres_probes.so")


def algo_bytes(T: int, N: int, D: int):
    """Bytes the operator must move (single pass, nothing materialised beyond
    the outputs): fwd reads sources and writes out + rstd + alpha; bwd reads
    sources, dout, rstd, alpha and writes dsources.  Per-call extras: w read
    (4D per call) and, for the backward, dw written (4D).  The backward's own
    workspace traffic (dw partial rows written and read back) is not counted
    here; workspace_traffic() gives it."""
    fwd = T * (2 * N * D + 2 * D + 8 * N)
    bwd = T * (4 * N * D + 2 * D + 8 * N)
    fwd_extra = 4 * D
    bwd_extra = 4 * D + 4 * D
    return fwd, bwd, fwd_extra, bwd_extra


def workspace_traffic(T: int, N: int, D: int) -> int:
    """Bytes one attnres_bwd call moves through its workspace (written plus
    read; not HBM bytes: a chunk's partial rows mostly stay in the Infinity
    Cache).  Where the split backward runs (ATTNRES_BWD_SPLIT(N, D)): the
    per-span dw partial rows (ceil(T/4) rows of D fp32) written and read back,
    the P = min(spans, 256) fold rows written by every chunk's fold, re-read by
    every later one and read by the final sum (no fold when P spans fill the
    rows: then the final sum reads the partial rows), and the ring slots the
    batch uses cleared; otherwise the min(T, 256) partial rows written and
    read."""
    import attention_residuals_depth_amd as ar

    if ar.bwd_split(N, D):
        groups = (T + 3) // 4
        chunks = (groups + 8191) // 8192
        P = min(groups, 256)
        K = (D + 1023) // 1024
        ring = min(T, 4096) * K * 2 * N * 8 if K > 1 else 0  # one slice per row: no ring
        fold = 4 * P * D * (2 * chunks) if groups > 256 else 0
        return 8 * groups * D + fold + ring
    return 8 * min(T, 256) * D


def kernel_source_hash() -> str:
    """Hash of the kernel source's code: comments and whitespace are dropped, so
    recorded counter traffic stays valid across comment edits and goes stale
    (reported as null) on any change to the code."""
    text = open(KERNEL_SRC, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode("utf-8")).hexdigest()[:16]


def traffic_file(T: int, N: int, D: int) -> str:
    return os.path.join(PROFILES, f"traffic_bwd_T{T}_N{N}_D{D}.json")


def load_traffic(T: int, N: int, D: int):
    """HBM bytes per attnres_bwd call from the committed rocprofv3 counter runs
    for this workload (FETCH_SIZE and WRITE_SIZE, calibrated against a copy of
    known size), used only while the kernel source is the one the counters
    were taken on; otherwise None."""
    try:
        rec = json.load(open(traffic_file(T, N, D)))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    if (rec.get("T"), rec.get("N"), rec.get("D")) != (T, N, D):
        return None
    return rec


def log(msg: str):
    """Progress on stderr (the JSON line is the only stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def make_inputs(wl, torch, dev, chunk: int = 8192):
    """The workload's sources, dout and w, generated on the host chunk by chunk
    (counter-based, so any token range is reproducible on its own) and copied
    into device tensors; the host arrays are kept for the oracle pass."""
    import numpy as np

    src_h = np.empty((wl.N, wl.T, wl.D), dtype=np.uint16)
    dout_h = np.empty((wl.T, wl.D), dtype=np.uint16)
    src = torch.empty((wl.N, wl.T, wl.D), dtype=torch.bfloat16, device=dev)
    dout = torch.empty((wl.T, wl.D), dtype=torch.bfloat16, device=dev)
    for t0 in range(0, wl.T, chunk):
        t1 = min(wl.T, t0 + chunk)
        wl.sources(t0, t1, out=src_h[:, t0:t1])  # row block i is contiguous in each source
        wl.dout(t0, t1, out=dout_h[t0:t1])
        src[:, t0:t1].view(torch.int16).copy_(torch.from_numpy(src_h[:, t0:t1].view(np.int16)))
        dout[t0:t1].view(torch.int16).copy_(torch.from_numpy(dout_h[t0:t1].view(np.int16)))
        if (t0 // chunk) % 4 == 3 or t1 == wl.T:
            log(f"inputs: tokens 0..{t1} of {wl.T} generated")
    w_h = wl.w()
    return src, torch.from_numpy(w_h).to(dev), dout, (src_h, w_h, dout_h)


def sample_tokens(T: int, n_random: int = 48, seed: int = 1):
    """First and last tokens, the first and last backward workgroup's first
    tokens, the start of the last (ragged) round of tokens, seeded random ones."""
    import numpy as np

    P = min(T, 256)
    edges = {0, 1, T - 2, T - 1, P - 1, P, 2 * P - 1}
    last_round = (T // P) * P if T % P else T - P
    edges.update({last_round, last_round - 1, last_round + 1})
    rnd = np.random.default_rng(seed).integers(0, T, size=n_random)
    return np.array(sorted({int(t) for t in edges if 0 <= t < T} | {int(t) for t in rnd}), dtype=np.int64)


def omp_threads() -> int:
    try:
        return int(ctypes.CDLL("libgomp.so.1").omp_get_max_threads())
    except OSError:
        return os.cpu_count() or 1


# Parity bars: relative L2 for out (5e-3), dsources and dw (1e-2), absolute for
# alpha (1e-5); rstd relative 1e-5 (an fp32 sum of D exact bf16 squares is
# good to ~1e-6 relative).
PARITY_BARS = {"out_rel_l2": 5e-3, "out_token_rel_l2": 5e-3, "alpha_max_abs": 1e-5, "rstd_max_rel": 1e-5,
               "dsrc_rel_l2": 1e-2, "dw_rel_l2": 1e-2}


class _Errors:
    """Error metrics accumulated over token chunks (torch CPU ops, float64)."""

    def __init__(self, torch):
        self.torch = torch
        self.v = {"out_err": 0.0, "out_ref": 0.0, "out_token_rel_l2": 0.0, "alpha_max_abs": 0.0, "rstd_max_rel": 0.0}

    def fwd_chunk(self, out_gpu_bits, rstd_gpu, alpha_gpu, o_out, o_rstd, o_alpha):
        import numpy as np

        torch = self.torch
        go = torch.from_numpy(np.ascontiguousarray(out_gpu_bits).view(np.int16)).view(torch.bfloat16).double()
        ro = torch.from_numpy(o_out)
        d2 = (go - ro).square_()
        self.v["out_err"] += float(d2.sum())
        self.v["out_ref"] += float(ro.square().sum())
        den = ro.square().sum(1).sqrt_()
        tok = d2.sum(1).sqrt_() / torch.where(den > 0, den, torch.ones_like(den))
        self.v["out_token_rel_l2"] = max(self.v["out_token_rel_l2"], float(tok.max()))
        self.v["alpha_max_abs"] = max(self.v["alpha_max_abs"], float(np.max(np.abs(alpha_gpu - o_alpha))))
        self.v["rstd_max_rel"] = max(self.v["rstd_max_rel"], float(np.max(np.abs(rstd_gpu - o_rstd) / o_rstd)))


def oracle_pass(wl, host, gpu, toks, torch, chunk: int = 4096):
    """The oracle, as it stands, over the whole workload in token chunks: the
    forward and the backward timed separately (monotonic clock around the
    oracle calls only), and the timed run's outputs compared with it: out,
    alpha, rstd on every token, dsources on the sampled tokens `toks`, dw
    summed over all chunks in token order.  Returns (record, parity)."""
    import numpy as np

    import oracle

    src_h, w_h, dout_h = host
    T, N, D = wl.T, wl.N, wl.D
    errs = _Errors(torch)
    t_fwd = t_bwd = 0.0
    o_dw = np.zeros(D)
    dsrc_err = dsrc_ref = 0.0
    pos = {int(t): j for j, t in enumerate(toks)}
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        xs = np.ascontiguousarray(src_h[:, t0:t1])
        c = time.perf_counter()
        o_out, o_rstd, o_alpha = oracle.fwd(xs, w_h, wl.eps)
        t_fwd += time.perf_counter() - c
        c = time.perf_counter()
        o_dsrc, dw_c = oracle.bwd(xs, w_h, wl.eps, dout_h[t0:t1])
        t_bwd += time.perf_counter() - c
        o_dw += dw_c
        errs.fwd_chunk(gpu["out_bits"][t0:t1], gpu["rstd"][t0:t1], gpu["alpha"][t0:t1], o_out, o_rstd, o_alpha)
        for t in [t for t in pos if t0 <= t < t1]:
            g = synth_bf16_to_f64(gpu["dsrc_bits"][:, pos[t]])
            r = o_dsrc[:, t - t0]
            dsrc_err += float(np.sum((g - r) ** 2))
            dsrc_ref += float(np.sum(r ** 2))
        del o_out, o_dsrc
        if (t0 // chunk) % 8 == 7 or t1 == T:
            log(f"oracle: tokens 0..{t1} of {T} (fwd {t_fwd:.1f} s, bwd {t_bwd:.1f} s)")
    e = {"out_rel_l2": (errs.v["out_err"] / errs.v["out_ref"]) ** 0.5, "out_token_rel_l2": errs.v["out_token_rel_l2"],
         "alpha_max_abs": errs.v["alpha_max_abs"], "rstd_max_rel": errs.v["rstd_max_rel"],
         "dsrc_rel_l2": (dsrc_err / dsrc_ref) ** 0.5,
         "dw_rel_l2": float(np.linalg.norm(gpu["dw"] - o_dw) / np.linalg.norm(o_dw))}
    e["within_bars"] = all(e[k] <= v for k, v in PARITY_BARS.items())
    e["compared"] = (f"out, alpha, rstd: all {T} tokens; dsources: {len(toks)} sampled tokens; "
                     f"dw: sum over all {T} tokens")
    cores = omp_threads()
    rec = {"value": T / (t_fwd + t_bwd), "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "fwd_tokens_per_s": T / t_fwd, "bwd_tokens_per_s": T / t_bwd,
           "sample": f"the whole workload ({T} tokens, N={N}, D={D}) in chunks of {chunk}, fp64, "
                     f"fwd {t_fwd:.1f} s + bwd {t_bwd:.1f} s on {cores} threads"}
    return rec, e


def synth_bf16_to_f64(bits):
    import numpy as np

    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def oracle_per_config(n_tokens: int = 2048):
    """The oracle's fwd and bwd timed separately on the first min(T, n_tokens)
    tokens of every workload (the N-sweep workload at N = 9)."""
    import oracle
    import synth

    rows = []
    for cfg in sorted(synth.WORKLOADS):
        wl = synth.workload(cfg, N=9 if cfg == 2 else None)
        S = min(wl.T, n_tokens)
        src, dout, w = wl.sources(0, S), wl.dout(0, S), wl.w()
        c = time.perf_counter()
        oracle.fwd(src, w, wl.eps)
        tf = time.perf_counter() - c
        c = time.perf_counter()
        oracle.bwd(src, w, wl.eps, dout)
        tb = time.perf_counter() - c
        rows.append({"workload": wl.name, "T": wl.T, "N": wl.N, "tokens_timed": S, "fwd_tokens_per_s": S / tf,
                     "bwd_tokens_per_s": S / tb})
    return rows


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence (hip_runtime_api.h)


def _hip_runtime():
    """The HIP runtime this process already uses (torch's libamdhip64, which
    the library resolves to as well), opened by path so that no second copy
    is loaded."""
    for line in open("/proc/self/maps"):
        path = line.split()[-1]
        if os.path.basename(path).startswith("libamdhip64.so"):
            return ctypes.CDLL(path)
    raise RuntimeError("the HIP runtime is not loaded in this process")


class TimingEvents:
    """HIP events recorded on a given stream and used only for timestamps.
    Created with hipEventDisableSystemFence: recording one then performs no
    system-scope fence, i.e. no L2 writeback and invalidation between the
    calls being timed (HIP documents the flag for timing-only events); the
    elapsed times are read after a full device synchronisation.  Falls back
    to default events if the runtime refuses the flag (`kind` says which)."""

    def __init__(self, n: int, fenceless: bool = True):
        self.hip = _hip_runtime()
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.kind = "hipEventDisableSystemFence" if fenceless else "default"
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE if fenceless else 0)
            if rc != 0 and fenceless and not self.ev:
                fenceless, self.kind = False, "default (hipEventDisableSystemFence refused)"
                rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), 0)
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            self.ev.append(e)

    def record(self, i: int, stream: int):
        rc = self.hip.hipEventRecord(self.ev[i], ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def ms(self, i: int, j: int) -> float:
        f = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(f), self.ev[i], self.ev[j])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return f.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def timed_steps(ar, torch, src, w, dout, eps, bufs, K, fenceless=True):
    """K steps (fwd then bwd) on the current stream.  One timing event sits
    between every two calls (2K + 1 in all): the event after a step's backward
    is the start of the next forward, so the split into fwd and bwd costs no
    extra marker per step."""
    out, rstd, alpha, dsrc, dw, ws = bufs
    stream = torch.cuda.current_stream().cuda_stream
    ev = TimingEvents(2 * K + 1, fenceless)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev.record(0, stream)
    for k in range(K):
        ar.attnres_fwd(src, w, eps, out=out, rstd=rstd, alpha=alpha)
        ev.record(2 * k + 1, stream)
        ar.attnres_bwd(dout, src, w, rstd, alpha, dsrc=dsrc, dw=dw, workspace=ws)
        ev.record(2 * k + 2, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = ev.ms(0, 2 * K)
    fwd_ms = sum(ev.ms(2 * k, 2 * k + 1) for k in range(K)) / K
    bwd_ms = sum(ev.ms(2 * k + 1, 2 * k + 2) for k in range(K)) / K
    kind = ev.kind
    ev.close()
    return total_ms, wall, fwd_ms, bwd_ms, kind


def alloc_buffers(ar, torch, N, T, D, dev):
    out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    rstd = torch.empty((T, N), dtype=torch.float32, device=dev)
    alpha = torch.empty((T, N), dtype=torch.float32, device=dev)
    dsrc = torch.empty((N, T, D), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((D,), dtype=torch.float32, device=dev)
    ws = torch.empty((ar.workspace_bytes(T, N, D),), dtype=torch.uint8, device=dev)
    return out, rstd, alpha, dsrc, dw, ws


def _fwd_bwd_ms(torch, flush, fwd, bwd, reps):
    """Median event times of fwd and bwd, caches flushed before each."""
    f_ms, b_ms = [], []
    stream = torch.cuda.current_stream().cuda_stream
    e = TimingEvents(4)
    for r in range(reps + 3):
        flush.zero_()
        e.record(0, stream)
        fwd()
        e.record(1, stream)
        flush.zero_()
        e.record(2, stream)
        bwd()
        e.record(3, stream)
        torch.cuda.synchronize()
        if r >= 3:
            f_ms.append(e.ms(0, 1))
            b_ms.append(e.ms(2, 3))
    e.close()
    return sorted(f_ms)[len(f_ms) // 2], sorted(b_ms)[len(b_ms) // 2]


def sweep(ar, torch, dev, reps=20):
    """Per-T (N=9) and per-N (T=32768) lines, fwd and bwd timed separately,
    caches flushed (a 512 MiB write) between reps; inputs are device-side
    random bf16 of the workload's scales (values do not affect timing).  Each
    line gives the stacked [N][T][D] calls and, as "interleaved", the same
    sources side by side per token ([T][N][D] cache, gradients likewise)
    through the per-source calls, and the peak allocated memory of the
    stacked case (sources, dout, w, outputs, saved state, dw, workspace)."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cases = [(9, T, 7168) for T in (1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072, 262144)]
    cases += [(N, 32768, 7168) for N in range(2, 9)]
    cases += [(9, 32768, D) for D in (4096, 12288, 16384)]  # other hidden sizes
    for N, T, D in cases:
        torch.cuda.synchronize()
        held = torch.cuda.memory_allocated()  # the flush buffer and whatever the caller still holds
        g = torch.Generator(device=dev)
        g.manual_seed(0)
        scale = torch.sqrt(1 + 12 * torch.arange(N, device=dev, dtype=torch.float32)).view(N, 1, 1)
        src = (torch.randn((N, T, D), device=dev, generator=g) * scale).to(torch.bfloat16)
        dout = torch.randn((T, D), device=dev, generator=g).to(torch.bfloat16)
        w = torch.randn(D, device=dev, generator=g) / D ** 0.5
        # peak allocated memory of the operator's own tensors (inputs, outputs,
        # workspace): from here on only they are allocated beyond `held`
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        bufs = alloc_buffers(ar, torch, N, T, D, dev)
        out, rstd, alpha, dsrc, dw, ws = bufs
        f, b = _fwd_bwd_ms(torch, flush, lambda: ar.attnres_fwd(src, w, 1e-6, out=out, rstd=rstd, alpha=alpha),
                           lambda: ar.attnres_bwd(dout, src, w, rstd, alpha, dsrc=dsrc, dw=dw, workspace=ws), reps)
        peak_gib = (torch.cuda.max_memory_allocated() - held) / 2**30
        del dsrc
        cache = src.permute(1, 0, 2).contiguous()  # [T][N][D]
        del src
        torch.cuda.empty_cache()
        dcache = torch.empty_like(cache)
        views = [cache[:, i] for i in range(N)]
        dviews = [dcache[:, i] for i in range(N)]
        fi, bi = _fwd_bwd_ms(torch, flush,
                             lambda: ar.attnres_fwd_sources(views, w, 1e-6, out=out, rstd=rstd, alpha=alpha),
                             lambda: ar.attnres_bwd_sources(dout, views, w, rstd, alpha, dsrcs=dviews, dw=dw,
                                                            workspace=ws), reps)
        fb, bb, fe, be = algo_bytes(T, N, D)
        line = {"sweep": True, "N": N, "T": T, "D": D, "fwd_ms": f, "bwd_ms": b,
                "fwd_GBps": (fb + fe) / f / 1e6, "bwd_GBps": (bb + be) / b / 1e6,
                "fwdbwd_tokens_per_s": T / ((f + b) * 1e-3),
                "fwdbwd_GBps": (fb + bb + fe + be) / (f + b) / 1e6,
                "fwdbwd_frac_of_8TBps": (fb + bb + fe + be) / (f + b) / 1e6 / HBM_PEAK_GBPS,
                "peak_alloc_GiB": peak_gib,
                "interleaved": {"fwd_ms": fi, "bwd_ms": bi, "fwd_GBps": (fb + fe) / fi / 1e6,
                                "bwd_GBps": (bb + be) / bi / 1e6, "fwdbwd_tokens_per_s": T / ((fi + bi) * 1e-3),
                                "fwdbwd_frac_of_8TBps": (fb + bb + fe + be) / (fi + bi) / 1e6 / HBM_PEAK_GBPS}}
        print(json.dumps(line), flush=True)
        del cache, dcache, views, dviews, dout, w, bufs, out, rstd, alpha, dw, ws
        torch.cuda.empty_cache()
    sweep_sources(ar, torch, dev, flush, reps)


def sweep_sources(ar, torch, dev, flush, reps, N=9, T=32768, D=7168):
    """Per-source calls (separately allocated sources and gradients) at T=32768,
    N=9: the forward, the overwriting backward, the accumulating backward (which
    also reads the old gradients: +2ND bytes per token), and the forward fused
    with the partial-sum update next to the unfused route (elementwise add, then
    the forward), both counted at the fused call's algorithmic bytes."""
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    srcs = [(torch.randn((T, D), device=dev, generator=g) * (1 + 12 * i) ** 0.5).to(torch.bfloat16) for i in range(N)]
    dout = torch.randn((T, D), device=dev, generator=g).to(torch.bfloat16)
    w = torch.randn(D, device=dev, generator=g) / D ** 0.5
    dsrcs = [torch.zeros((T, D), dtype=torch.bfloat16, device=dev) for _ in range(N)]
    out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    rstd = torch.empty((T, N), dtype=torch.float32, device=dev)
    alpha = torch.empty((T, N), dtype=torch.float32, device=dev)
    dw = torch.empty((D,), dtype=torch.float32, device=dev)
    ws = torch.empty((ar.workspace_bytes(T, N, D),), dtype=torch.uint8, device=dev)
    fb, bb, fe, be = algo_bytes(T, N, D)
    calls = {
        "fwd_sources": (lambda: ar.attnres_fwd_sources(srcs, w, 1e-6, out=out, rstd=rstd, alpha=alpha), fb + fe),
        "bwd_sources": (lambda: ar.attnres_bwd_sources(dout, srcs, w, rstd, alpha, dsrcs=dsrcs, dw=dw, workspace=ws),
                        bb + be),
        "bwd_sources_accumulate": (lambda: ar.attnres_bwd_sources(dout, srcs, w, rstd, alpha, dsrcs=dsrcs,
                                                                  accumulate=True, dw=dw, workspace=ws),
                                   bb + be + T * 2 * N * D),
    }
    # fp32 gradients: written (2ND more bytes than bf16) and accumulated (4ND more read)
    g32 = [torch.zeros((T, D), dtype=torch.float32, device=dev) for _ in range(N)]
    calls["bwd_sources_f32"] = (lambda: ar.attnres_bwd_sources(dout, srcs, w, rstd, alpha, dsrcs=g32, dw=dw,
                                                               workspace=ws), bb + be + T * 2 * N * D)
    calls["bwd_sources_f32_accumulate"] = (lambda: ar.attnres_bwd_sources(dout, srcs, w, rstd, alpha, dsrcs=g32,
                                                                          accumulate=True, dw=dw, workspace=ws),
                                           bb + be + T * 6 * N * D)
    # partial-sum update fused into the forward (last source = bf16(p + y)),
    # against the unfused route: a separate elementwise add, then the forward
    p = srcs[-1].clone()
    y = (torch.randn((T, D), device=dev, generator=g) * 0.5).to(torch.bfloat16)
    upd_bytes = T * (2 * (N + 1) * D + 4 * D + 8 * N) + 4 * D

    def unfused():
        torch.add(p, y, out=p)
        ar.attnres_fwd_sources(srcs[:-1] + [p], w, 1e-6, out=out, rstd=rstd, alpha=alpha)

    calls["fwd_update_fused"] = (lambda: ar.attnres_fwd_update(srcs[:-1], p, y, w, 1e-6, out=out, rstd=rstd,
                                                               alpha=alpha), upd_bytes)
    calls["fwd_update_unfused"] = (unfused, upd_bytes)
    # the same sources side by side per token ([T][N][D] cache, row pitch N*D),
    # gradients into a cache of the same layout
    cache = torch.stack(srcs, dim=1)
    views = [cache[:, i] for i in range(N)]
    dcache = torch.empty_like(cache)
    dviews = [dcache[:, i] for i in range(N)]
    calls["fwd_interleaved"] = (lambda: ar.attnres_fwd_sources(views, w, 1e-6, out=out, rstd=rstd, alpha=alpha),
                                fb + fe)
    calls["bwd_interleaved"] = (lambda: ar.attnres_bwd_sources(dout, views, w, rstd, alpha, dsrcs=dviews, dw=dw,
                                                               workspace=ws), bb + be)
    for name, (fn, nbytes) in calls.items():
        m = _median_ms(torch, flush, fn, reps)
        print(json.dumps({"sweep": True, "call": name, "N": N, "T": T, "D": D, "ms": m,
                          "GBps": nbytes / m / 1e6, "frac_of_8TBps": nbytes / m / 1e6 / HBM_PEAK_GBPS}), flush=True)
    del srcs, dsrcs, dout, p, y, cache, views, dcache, dviews, g32
    torch.cuda.empty_cache()
    sweep_decode(ar, torch, dev, flush)


def _median_ms(torch, flush, fn, reps):
    """Median event time of fn over reps calls, caches flushed before each."""
    ms = []
    stream = torch.cuda.current_stream().cuda_stream
    e = TimingEvents(2)
    for r in range(reps + 3):
        flush.zero_()
        e.record(0, stream)
        fn()
        e.record(1, stream)
        torch.cuda.synchronize()
        if r >= 3:
            ms.append(e.ms(0, 1))
    e.close()
    return sorted(ms)[len(ms) // 2]


def sweep_decode(ar, torch, dev, flush, N=9, D=7168):
    """Decoding-size batches through attnres_fwd_decode (no saved state): one
    flushed call (latency, inputs in HBM) and the mean of 200 back-to-back calls
    (inputs cache-resident; at these sizes the host's call rate bounds it)."""
    for T in (1, 8, 64, 256, 1024):
        g = torch.Generator(device=dev)
        g.manual_seed(0)
        srcs = [(torch.randn((T, D), device=dev, generator=g) * (1 + 12 * i) ** 0.5).to(torch.bfloat16)
                for i in range(N)]
        w = torch.randn(D, device=dev, generator=g) / D ** 0.5
        out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
        fn = lambda: ar.attnres_fwd_decode(srcs, w, 1e-6, out=out)
        cold_us = _median_ms(torch, flush, fn, 20) * 1e3
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        e = TimingEvents(2)
        stream = torch.cuda.current_stream().cuda_stream
        e.record(0, stream)
        for _ in range(200):
            fn()
        e.record(1, stream)
        torch.cuda.synchronize()
        warm_us = e.ms(0, 1) / 200 * 1e3
        e.close()
        print(json.dumps({"sweep": True, "call": "fwd_decode", "N": N, "T": T, "D": D, "cold_us": cold_us,
                          "back_to_back_us": warm_us}), flush=True)


class Probes:
    """ctypes view of libattnres_probes (bandwidth ceilings; not the operator)."""

    def __init__(self):
        if not os.path.exists(PROBE_LIB):
            raise RuntimeError(f"{PROBE_LIB} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(PROBE_LIB)
        vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
        pp = ctypes.POINTER(ctypes.c_void_p)
        lib.attnres_probe_read.argtypes = [vp, sz, vp, vp]
        lib.attnres_probe_write.argtypes = [vp, sz, vp]
        lib.attnres_probe_copy.argtypes = [vp, vp, sz, vp]
        lib.attnres_probe_fwd_pattern.argtypes = [pp, i32, i64, i32, vp, vp]
        lib.attnres_probe_bwd_pattern.argtypes = [pp, vp, i32, i64, i32, pp, vp]
        lib.attnres_probe_split_bwd_pattern.argtypes = [pp, vp, i32, i64, i32, pp, vp, vp]
        self.lib = lib

    @staticmethod
    def check(rc, name):
        if rc != 0:
            raise RuntimeError(f"{name} returned {rc}")


def ceilings(torch, dev, src, dout, out, dsrc, reps: int = 5, nbytes: int = 4 << 30):
    """Median GB/s of the probe kernels on this device: plain read, write and
    copy streams of `nbytes` (one 4 KiB chunk per workgroup, nontemporal), and
    the operator's forward and backward access patterns on the workload's own
    buffers (same rows, same launch shapes, no arithmetic; the backward both as
    the one-token kernel and as the split kernel walk the rows).  Overwrites
    out and dsrc."""
    pr = Probes()
    stream = torch.cuda.current_stream().cuda_stream
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    N, T, D = src.shape
    part = torch.empty((min((T + 3) // 4, 8192), D), dtype=torch.float32, device=dev)
    srcs = (ctypes.c_void_p * N)(*[src[i].data_ptr() for i in range(N)])
    dsrcs = (ctypes.c_void_p * N)(*[dsrc[i].data_ptr() for i in range(N)])
    calls = {
        "read": (lambda: pr.check(pr.lib.attnres_probe_read(a.data_ptr(), nbytes, sink.data_ptr(), stream), "read"),
                 nbytes),
        "write": (lambda: pr.check(pr.lib.attnres_probe_write(b.data_ptr(), nbytes, stream), "write"), nbytes),
        "copy": (lambda: pr.check(pr.lib.attnres_probe_copy(a.data_ptr(), b.data_ptr(), nbytes, stream), "copy"),
                 2 * nbytes),
        "fwd_pattern": (lambda: pr.check(pr.lib.attnres_probe_fwd_pattern(srcs, N, T, D, out.data_ptr(), stream),
                                         "fwd_pattern"), T * (2 * N * D + 2 * D)),
        "bwd_pattern": (lambda: pr.check(pr.lib.attnres_probe_bwd_pattern(srcs, dout.data_ptr(), N, T, D, dsrcs,
                                                                          stream), "bwd_pattern"),
                        T * (4 * N * D + 2 * D)),
        # the split backward's pattern, counted at the same bytes (its partial rows are not counted)
        "split_bwd_pattern": (lambda: pr.check(pr.lib.attnres_probe_split_bwd_pattern(
            srcs, dout.data_ptr(), N, T, D, dsrcs, part.data_ptr(), stream), "split_bwd_pattern"),
                              T * (4 * N * D + 2 * D)),
    }
    res = {}
    ev = TimingEvents(2)
    for name, (fn, moved) in calls.items():
        if name.endswith("pattern") and D > 8192:
            continue
        ms = []
        for r in range(reps + 2):
            ev.record(0, stream)
            fn()
            ev.record(1, stream)
            torch.cuda.synchronize()
            if r >= 2:
                ms.append(ev.ms(0, 1))
        res[name] = moved / (sorted(ms)[len(ms) // 2] * 1e-3) / 1e9
    ev.close()
    del a, b, part
    torch.cuda.empty_cache()
    return res


def block_batched(ar, torch, dev, T: int = 32768, n: int = 8, L: int = 24, D: int = 7168, reps: int = 5):
    """One block's forwards three ways (the model's last block: n = 8 shared
    sources -- embedding and 7 completed block sums -- plus the partial sum,
    L = 24 sub-layers): L plain per-source forwards; one block-scores pass
    (MFMA) followed by L forwards from those scores; and block scores, one
    block-sums pass (the shared sources' part of every sub-layer's weighted
    sum, fp32 sub-layer-major and token-major, and in the 24-bit element
    format sub-layer-major) and L merged forwards that read only the shared
    sum and the partial sum.  Then a model's block, where the partial sum
    advances before every sub-layer: L plain forwards with the fused update
    against block scores, 24-bit block sums and L merged forwards with it.  Median of `reps`
    whole-block timings, each preceded by a 512 MiB cache flush; per-call
    times from the same runs.  Device-side random inputs of the workload's
    scales (values do not change the timing)."""
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    N = n + 1
    srcs = [(torch.randn((T, D), device=dev, generator=g) * (1 + 12 * i) ** 0.5).to(torch.bfloat16) for i in range(N)]
    W = torch.randn((L, D), device=dev, generator=g) / D ** 0.5
    out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    rstd = torch.empty((T, N), dtype=torch.float32, device=dev)
    alpha = torch.empty((T, N), dtype=torch.float32, device=dev)
    rb = torch.empty((T, n), dtype=torch.float32, device=dev)
    zb = torch.empty((L, T, n), dtype=torch.float32, device=dev)
    ws = torch.empty((ar.block_scores_workspace_bytes(L, D),), dtype=torch.uint8, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    ev = TimingEvents(L + 3)
    U = None

    def plain():
        ev.record(0, stream)
        for l in range(L):
            ar.attnres_fwd_sources(srcs, W[l], 1e-6, out=out, rstd=rstd, alpha=alpha)
            ev.record(l + 1, stream)

    def batched():
        ev.record(0, stream)
        ar.attnres_block_scores(srcs[:n], W, 1e-6, rstd=rb, z=zb, workspace=ws)
        ev.record(1, stream)
        for l in range(L):
            ar.attnres_fwd_scored(srcs, zb[l], rb, W[l], 1e-6, out=out, rstd=rstd, alpha=alpha)
            ev.record(l + 2, stream)

    def merged(token_major, u_format="f32"):
        def run():
            ev.record(0, stream)
            ar.attnres_block_scores(srcs[:n], W, 1e-6, rstd=rb, z=zb, workspace=ws)
            ev.record(1, stream)
            ar.attnres_block_sums(srcs[:n], zb, U=U, token_major=token_major, u_format=u_format)
            ev.record(2, stream)
            for l in range(L):
                ar.attnres_fwd_merged(U[:, l] if token_major else U[l], srcs[n], zb[l], rb, W[l], 1e-6, out=out,
                                      rstd=rstd, alpha=alpha)
                ev.record(l + 3, stream)
        return run

    def timed(fn, last, marks, prep=None):
        tot, parts = [], {m: [] for m in marks}
        for r in range(reps + 2):
            if prep is not None:
                prep()
            flush.zero_()
            fn()
            torch.cuda.synchronize()
            if r >= 2:
                tot.append(ev.ms(0, last))
                for m in marks:
                    parts[m].append(ev.ms(m[0], m[1]))
        med = lambda v: sorted(v)[len(v) // 2]
        return med(tot), {m: med(v) for m, v in parts.items()}

    plain_ms, pp = timed(plain, L, [(0, 1)])
    batched_ms, bp = timed(batched, L + 1, [(0, 1)])
    scores_ms = bp[(0, 1)]
    merged_res = {}
    for tm, fmt in ((False, "f32"), (True, "f32"), (False, "f24")):
        if fmt == "f24":
            U = torch.empty((L, T, D, 3), dtype=torch.uint8, device=dev)
        else:
            U = torch.empty((T, L, D) if tm else (L, T, D), dtype=torch.float32, device=dev)
        ms, mp = timed(merged(tm, fmt), L + 2, [(1, 2), (2, L + 2)])
        merged_res[(tm, fmt)] = (ms, mp[(1, 2)], mp[(2, L + 2)] / L)
        del U
        U = None
        torch.cuda.empty_cache()
    # A model's block: before each sub-layer the partial sum advances by the
    # previous sub-layer's output, so the pair that matters is 24 plain
    # forwards with the fused update against block scores + 24-bit block sums
    # + 24 merged forwards with the fused update.  The partial sum is restored
    # before each timed block, ahead of the flush.
    y = (torch.randn((T, D), device=dev, generator=g) * 0.3).to(torch.bfloat16)
    p0 = srcs[n].clone()
    p = srcs[n].clone()
    U = torch.empty((L, T, D, 3), dtype=torch.uint8, device=dev)

    def restore():
        p.copy_(p0)

    def plain_update():
        ev.record(0, stream)
        for l in range(L):
            ar.attnres_fwd_update(srcs[:n], p, y, W[l], 1e-6, out=out, rstd=rstd, alpha=alpha)
            ev.record(l + 1, stream)

    def merged_update():
        ev.record(0, stream)
        ar.attnres_block_scores(srcs[:n], W, 1e-6, rstd=rb, z=zb, workspace=ws)
        ev.record(1, stream)
        ar.attnres_block_sums(srcs[:n], zb, U=U, u_format="f24")
        ev.record(2, stream)
        for l in range(L):
            ar.attnres_fwd_merged(U[l], p, zb[l], rb, W[l], 1e-6, delta=y, out=out, rstd=rstd, alpha=alpha)
            ev.record(l + 3, stream)

    pu_ms, _ = timed(plain_update, L, [(0, 1)], prep=restore)
    mu_ms, mup = timed(merged_update, L + 2, [(1, 2), (2, L + 2)], prep=restore)
    model_block = {"plain_update_block_ms": pu_ms, "merged_f24_update_block_ms": mu_ms,
                   "vs_plain_update": pu_ms / mu_ms, "block_sums_ms": mup[(1, 2)],
                   "merged_update_fwd_ms": mup[(2, L + 2)] / L}
    del U, y, p0, p
    U = None
    torch.cuda.empty_cache()
    ev.close()
    scored_ms = (batched_ms - scores_ms) / L
    scores_bytes = T * n * (2 * D + 4) + L * T * n * 4 + 4 * L * D  # sources read; rstd, z written; W read
    fwd_bytes = T * (2 * N * D + 2 * D + 8 * N) + 4 * D
    scored_bytes = fwd_bytes + T * (N - 1) * 8  # + the given scores and rstd
    sums_bytes = T * n * 2 * D + L * T * n * 4 + L * T * D * 4  # shared sources and z read; U written
    merged_bytes = T * (4 * D + 2 * D + 2 * D + 8 * (N - 1) + 8 * N) + 4 * D  # U, p read; out written; scores, state
    rec = {"T": T, "n_shared": n, "N": N, "L": L, "D": D,
           "plain_block_ms": plain_ms, "batched_block_ms": batched_ms, "batched_vs_plain": plain_ms / batched_ms,
           "plain_fwd_ms": plain_ms / L, "first_plain_fwd_ms": pp[(0, 1)],
           "block_scores_ms": scores_ms, "block_scores_GBps": scores_bytes / scores_ms / 1e6,
           "block_scores_TFLOPs": 2.0 * T * n * D * L / scores_ms / 1e9,
           "block_scores_mfma_TFLOPs": 2.0 * T * n * D * (16 * ((L + 15) // 16)) * 3 / scores_ms / 1e9,
           "scored_fwd_ms": scored_ms, "scored_fwd_GBps": scored_bytes / scored_ms / 1e6,
           "plain_fwd_GBps": fwd_bytes / (plain_ms / L) / 1e6,
           "U_GiB": L * T * D * 4 / 2 ** 30}
    for tm, fmt, key in ((False, "f32", "l_major"), (True, "f32", "t_major"), (False, "f24", "l_major_f24")):
        ms, sums_ms, mfwd_ms = merged_res[(tm, fmt)]
        eb = 3 if fmt == "f24" else 4  # bytes per element of U
        sb = sums_bytes - L * T * D * (4 - eb)
        mb = merged_bytes - T * D * (4 - eb)
        rec[f"merged_{key}"] = {"block_ms": ms, "vs_plain": plain_ms / ms, "block_sums_ms": sums_ms,
                                "block_sums_GBps": sb / sums_ms / 1e6, "merged_fwd_ms": mfwd_ms,
                                "merged_fwd_GBps": mb / mfwd_ms / 1e6}
    # one sub-layer's merged forward with the fused partial-sum update, against a
    # separate bf16 add followed by the merged forward (median of 11 calls)
    U = torch.empty((L, T, D), dtype=torch.float32, device=dev)
    ar.attnres_block_scores(srcs[:n], W, 1e-6, rstd=rb, z=zb, workspace=ws)
    ar.attnres_block_sums(srcs[:n], zb, U=U)
    y = (torch.randn((T, D), device=dev, generator=g) * 0.3).to(torch.bfloat16)
    p = srcs[n].clone()

    def fused():
        ar.attnres_fwd_merged(U[5], p, zb[5], rb, W[5], 1e-6, delta=y, out=out, rstd=rstd, alpha=alpha)

    def unfused():
        torch.add(p, y, out=p)
        ar.attnres_fwd_merged(U[5], p, zb[5], rb, W[5], 1e-6, out=out, rstd=rstd, alpha=alpha)

    upd_bytes = T * (4 * D + 8 * D + 8 * (N - 1) + 8 * N) + 4 * D  # U, p, y read; p, out written
    f_ms, u_ms = _median_ms(torch, flush, fused, 11), _median_ms(torch, flush, unfused, 11)
    rec["merged_update"] = {"fused_ms": f_ms, "fused_GBps": upd_bytes / f_ms / 1e6, "add_then_merged_ms": u_ms}
    del U, y, p
    rec["model_block"] = model_block
    rec["reps"] = f"median of {reps}, 512 MiB flush before each block"
    del srcs, W, out, rstd, alpha, rb, zb, ws, flush
    torch.cuda.empty_cache()
    return rec


def flushed_calls(torch, dev, fwd, bwd, reps: int = 10):
    """Median event times of fwd and of bwd, each preceded by a 512 MiB write
    that evicts the L2 and the 256 MB Infinity Cache."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    f, b = _fwd_bwd_ms(torch, flush, fwd, bwd, reps)
    del flush
    torch.cuda.empty_cache()
    return f, b


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=DEFAULT_WORKLOAD, choices=[0, 1, 2, 3, 4],
                    help="bench-line workload (default 3: T=131072, N=9, peaked softmax); 2 runs at N=9")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true")
    ap.add_argument("--default-events", action="store_true",
                    help="time with default HIP events (a system-scope fence at every marker) instead of "
                         "timing-only events, for comparison")
    ap.add_argument("--decode", action="store_true",
                    help="only the decoding-size forward calls (T = 1..1024), for latency profiles")
    ap.add_argument("--block", action="store_true",
                    help="only the block-batched measurement (one JSON line), for profiles")
    ap.add_argument("--no-block", action="store_true", help="skip the block-batched measurement")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the operator is token-local and the library has no "
              "multi-GPU path (--gpus must be 1)", file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import attention_residuals_depth_amd as ar
    import synth

    dev = torch.device("cuda:0")
    ar.library()
    if args.decode:
        sweep_decode(ar, torch, dev, torch.empty(512 << 20, dtype=torch.uint8, device=dev))
        return
    if args.block:
        print(json.dumps({"block_batched_scores": block_batched(ar, torch, dev)}), flush=True)
        return
    wl = synth.workload(args.workload, N=9 if args.workload == 2 else None)
    T, N, D = wl.T, wl.N, wl.D
    log(f"workload {wl.name}: T={T} N={N} D={D}")
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    src, w, dout, host = make_inputs(wl, torch, dev)
    bufs = alloc_buffers(ar, torch, N, T, D, dev)
    out, rstd, alpha, dsrc, dw, ws = bufs

    fenceless = not args.default_events
    log(f"{args.warmup} warm-up steps, then {args.steps} timed steps")
    timed_steps(ar, torch, src, w, dout, wl.eps, bufs, max(args.warmup, 1), fenceless)
    total_ms, wall, fwd_ms, bwd_ms, ev_kind = timed_steps(ar, torch, src, w, dout, wl.eps, bufs, args.steps,
                                                          fenceless)
    peak_gib = (torch.cuda.max_memory_allocated() - base) / 2**30
    # the timed run's outputs (every step computes the same batch), kept for the parity check
    toks = sample_tokens(T)
    tk = torch.from_numpy(toks).to(dev)
    gpu = {"out_bits": out.view(torch.int16).cpu().numpy().view(np.uint16),
           "rstd": rstd.cpu().double().numpy(), "alpha": alpha.cpu().double().numpy(),
           "dsrc_bits": dsrc[:, tk].contiguous().view(torch.int16).cpu().numpy().view(np.uint16),
           "dw": dw.cpu().double().numpy()}

    log("flushed per-call timing")
    f_fl, b_fl = flushed_calls(torch, dev, lambda: ar.attnres_fwd(src, w, wl.eps, out=out, rstd=rstd, alpha=alpha),
                               lambda: ar.attnres_bwd(dout, src, w, rstd, alpha, dsrc=dsrc, dw=dw, workspace=ws))
    ceil = None
    if not args.no_probes:
        log("bandwidth ceilings (probe kernels)")
        ceil = ceilings(torch, dev, src, dout, out, dsrc)
    blk = None
    if not args.no_block:
        log("block-batched scores and sums vs plain forwards (T=32768, 8 shared sources, 24 sub-layers)")
        blk = block_batched(ar, torch, dev)

    ms_step = total_ms / args.steps
    fb, bb, fe, be = algo_bytes(T, N, D)
    step_gbps = (fb + bb + fe + be) / (ms_step * 1e-3) / 1e9
    bwd_gbps = (bb + be) / (bwd_ms * 1e-3) / 1e9
    fwd_gbps = (fb + fe) / (fwd_ms * 1e-3) / 1e9
    traffic = load_traffic(T, N, D)

    result = {
        "metric": METRIC,
        "value": T * args.steps / (total_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "accumulate": "f32",
        "data": ("synthetic (seeded counter-based generator; sources N(0,1)*sqrt(1+12i), "
                 f"w N(0,{wl.w_std if wl.w_std is not None else '1/sqrt(D)'}), dout N(0,1))"),
        "config": {"workload": wl.name, "T": T, "N": N, "D": D, "eps": wl.eps, "layout": "stacked [N][T][D]",
                   "parallelism": "single GPU"},
        "achieved_GBps": step_gbps,
        "hbm_frac": step_gbps / HBM_PEAK_GBPS,
        "fwd_ms": fwd_ms,
        "bwd_ms": bwd_ms,
        "fwd_GBps": fwd_gbps,
        "bwd_GBps": bwd_gbps,
        "flushed": {"fwd_ms": f_fl, "bwd_ms": b_fl, "fwd_GBps": (fb + fe) / f_fl / 1e6,
                    "bwd_GBps": (bb + be) / b_fl / 1e6, "fwdbwd_GBps": (fb + bb + fe + be) / (f_fl + b_fl) / 1e6,
                    "fwdbwd_tokens_per_s": T / ((f_fl + b_fl) * 1e-3), "reps": "median of 10"},
        "wall_s_timed": wall,
        "timing_events": ev_kind,
        "peak_alloc_GiB": peak_gib,
        "pages_peak_alloc_GiB_at_128K": PAGES_PEAK_GIB_128K,
        "ceilings_GBps": ceil,
        "block_batched_scores": blk,
        "bwd_workspace_bytes_moved": workspace_traffic(T, N, D),
        "roofline": {
            "kernel": "attnres_bwd (one call: ring clear, bwd_split_kernel, dw_fold_kernel, dw_reduce_kernel)",
            "bound": "hbm",
            "achieved": bwd_gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": bwd_gbps / HBM_PEAK_GBPS,
            "traffic": traffic["bytes_per_call"] if traffic else None,
        },
    }
    if not args.no_cpu_baseline:
        log("oracle pass on the host (fwd and bwd timed separately)")
        rec, parity = oracle_pass(wl, host, gpu, toks, torch)
        rec["per_workload_sample"] = oracle_per_config()
        result["cpu_baseline"] = rec
        result["parity"] = parity
    print(json.dumps(result), flush=True)
    if args.sweep:
        del src, dout, bufs, out, rstd, alpha, dsrc, dw, ws, host, gpu
        torch.cuda.empty_cache()
        sweep(ar, torch, dev)


if __name__ == "__main__":
    main()

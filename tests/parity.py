"""Helpers shared by the GPU parity tests (not a test module).

Inputs come from the seeded generator (``synth``); the expected values come
from the fp64 oracle (``oracle``) on the very same bytes.  The device path is
reached only through the C ABI (``attention_residuals_depth_amd``).
"""
from __future__ import annotations

import numpy as np
import torch

import attention_residuals_depth_amd as ar
import oracle
import synth

# Tolerances.  out, alpha, dsources and dw: the operator's acceptance bounds
# (relative L2 5e-3 forward and 1e-2 gradients, 1e-5 absolute on alpha);
# rstd's is derived: an fp32 sum of D <= 16384 exact bf16 squares carries a
# relative error below ~(log2 D + 8) * 2^-24 ~ 1.3e-6, and the square root and
# reciprocal add < 1 ulp each, so 1e-5 relative leaves a wide margin.
TOL_OUT_REL_L2 = 5e-3
TOL_ALPHA_ABS = 1e-5
TOL_RSTD_REL = 1e-5
TOL_DSRC_REL_L2 = 1e-2
TOL_DW_REL_L2 = 1e-2

DEV = "cuda:0"


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def bf16_dev_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().double().numpy()


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    nb = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b)) / (nb if nb > 0 else 1.0)


def sources_to_device(wl: synth.Workload, chunk: int = 4096) -> torch.Tensor:
    """Generate the workload's sources chunk by chunk straight into a device tensor."""
    dev = torch.empty((wl.N, wl.T, wl.D), dtype=torch.bfloat16, device=DEV)
    buf = np.empty((chunk, wl.D), dtype=np.uint16)
    scales = wl.source_scales()
    for i in range(wl.N):
        for t0 in range(0, wl.T, chunk):
            n = min(chunk, wl.T - t0)
            synth.rows_bf16(n, wl.D, wl.seed, synth.STREAM_SRC0 + i, t0, float(scales[i]), wl.channel_multipliers(i),
                            out=buf[:n])
            dev[i, t0:t0 + n].copy_(torch.from_numpy(buf[:n].view(np.int16)).view(torch.bfloat16))
    return dev


def dout_to_device(wl: synth.Workload, chunk: int = 16384) -> torch.Tensor:
    dev = torch.empty((wl.T, wl.D), dtype=torch.bfloat16, device=DEV)
    for t0 in range(0, wl.T, chunk):
        t1 = min(wl.T, t0 + chunk)
        dev[t0:t1].copy_(to_dev_bf16(wl.dout(t0, t1)))
    return dev


def token_rows(wl: synth.Workload, tokens: np.ndarray):
    """Host sources [N][len(tokens)][D] and dout [len(tokens)][D] of the given tokens."""
    src = np.empty((wl.N, len(tokens), wl.D), dtype=np.uint16)
    g = np.empty((len(tokens), wl.D), dtype=np.uint16)
    for j, t in enumerate(tokens):
        src[:, j:j + 1] = wl.sources(int(t), int(t) + 1)
        g[j:j + 1] = wl.dout(int(t), int(t) + 1)
    return src, g


def check_tokens(errs: dict, name: str, gpu: dict, ref: dict):
    """Record the error metrics of one comparison into errs[name]."""
    e = {
        "out_rel_l2": rel_l2(gpu["out"], ref["out"]),
        "alpha_max_abs": float(np.abs(gpu["alpha"] - ref["alpha"]).max()),
        "rstd_max_rel": float((np.abs(gpu["rstd"] - ref["rstd"]) / np.abs(ref["rstd"])).max()),
    }
    if "dsrc" in ref:
        e["dsrc_rel_l2"] = rel_l2(gpu["dsrc"], ref["dsrc"])
    if "dw" in ref:
        e["dw_rel_l2"] = rel_l2(gpu["dw"], ref["dw"])
    errs[name] = e
    return e


def within_tolerance(e: dict) -> bool:
    ok = e["out_rel_l2"] <= TOL_OUT_REL_L2 and e["alpha_max_abs"] <= TOL_ALPHA_ABS and e["rstd_max_rel"] <= TOL_RSTD_REL
    if "dsrc_rel_l2" in e:
        ok = ok and e["dsrc_rel_l2"] <= TOL_DSRC_REL_L2
    if "dw_rel_l2" in e:
        ok = ok and e["dw_rel_l2"] <= TOL_DW_REL_L2
    return ok


def run_gpu(src_d, w_d, eps, dout_d):
    out, rstd, alpha = ar.attnres_fwd(src_d, w_d, eps)
    dsrc, dw = ar.attnres_bwd(dout_d, src_d, w_d, rstd, alpha)
    torch.cuda.synchronize()
    return out, rstd, alpha, dsrc, dw


def full_compare(wl: synth.Workload):
    """Run fwd+bwd on the whole workload and compare every output with the oracle."""
    src = wl.sources()
    w = wl.w()
    dout = wl.dout()
    out, rstd, alpha, dsrc, dw = run_gpu(to_dev_bf16(src), torch.from_numpy(w).to(DEV), wl.eps, to_dev_bf16(dout))
    o_out, o_rstd, o_alpha = oracle.fwd(src, w, wl.eps)
    o_dsrc, o_dw = oracle.bwd(src, w, wl.eps, dout)
    gpu = dict(out=bf16_dev_to_f64(out), rstd=rstd.cpu().double().numpy(), alpha=alpha.cpu().double().numpy(),
               dsrc=bf16_dev_to_f64(dsrc), dw=dw.cpu().double().numpy())
    ref = dict(out=o_out, rstd=o_rstd, alpha=o_alpha, dsrc=o_dsrc, dw=o_dw)
    return gpu, ref


def sample_tokens(T: int, n_random: int = 40, seed: int = 1) -> np.ndarray:
    """First and last tokens, the first and last backward workgroup's first
    tokens, the start of the last (ragged) round of tokens, and seeded random
    tokens."""
    P = min(T, ar.DW_PARTIALS)
    edges = {0, 1, T - 2, T - 1, P - 1, P, 2 * P - 1}
    last_round = (T // P) * P if T % P else T - P
    edges.update({last_round, last_round - 1, last_round + 1})
    rnd = np.random.default_rng(seed).integers(0, T, size=n_random)
    return np.array(sorted({int(t) for t in edges if 0 <= t < T} | {int(t) for t in rnd}), dtype=np.int64)

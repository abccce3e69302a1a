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


def check_tokens(errs: dict, name: str, gpu: dict, ref: dict, inputs=None):
    """Record the error metrics of one comparison into errs[name].  With
    inputs = (x_bits [N][n][D], g_bits [n][D], w) of the compared tokens, every
    element of out and dsrc is also checked against its arithmetic error bound
    and every token against the relative L2 bars."""
    e = {
        "out_rel_l2": rel_l2(gpu["out"], ref["out"]),
        "alpha_max_abs": float(np.abs(gpu["alpha"] - ref["alpha"]).max()),
        "rstd_max_rel": float((np.abs(gpu["rstd"] - ref["rstd"]) / np.abs(ref["rstd"])).max()),
        "out_token_rel_l2": per_token_rel_l2(gpu["out"], ref["out"], 0),
    }
    if "dsrc" in ref:
        e["dsrc_rel_l2"] = rel_l2(gpu["dsrc"], ref["dsrc"])
        e["dsrc_token_rel_l2"] = per_token_rel_l2(gpu["dsrc"], ref["dsrc"], 1)
    if "dw" in ref:
        e["dw_rel_l2"] = rel_l2(gpu["dw"], ref["dw"])
    if inputs is not None:
        x_bits, g_bits, w = inputs
        e.update(elementwise_ratios(x_bits, g_bits, w, gpu, ref, device=DEV))
    errs[name] = e
    return e


# ----------------------------------------------------------------------------
# Element-by-element bounds
# ----------------------------------------------------------------------------
# The whole-tensor relative L2 above would let a few wrong elements through (one
# wrong 16-byte vector in a 4096-token batch moves out's rel-L2 by ~5%).  So
# every compared element of out and dsources must also lie within an error
# bound derived from the arithmetic the kernels perform:
#
#   out'_d  = bf16( fl( sum_i a'_i x_id ) ), a' the GPU's saved alpha (the very
#             values its weighted sum used):
#             |out' - out| <= ulp/2 + sum_i |a'_i - a_i||x_id| + G_N sum_i a'_i |x_id|
#   dx'_id  = bf16( fma(c1', fma(-k', x_id, w_d), a'_i g_d) ) with c1 = dz r,
#             k = z r / D formed in fp32 from the dots g.x_i and w.x_i (fp32 tree
#             sums: error <= G_D * sum_d |terms|), the saved r' and a'; the
#             first-order propagation of those errors gives the bound below,
#             doubled to cover second-order terms.
#
# G_n = n u / (1 - n u) with u = 2^-24; G_D uses 64 for the depth of the fp32
# summation trees of a D-long dot (at most ~40 roundings along any path for
# D <= 16384).  ulp is the bf16 spacing at max(|ref|, |gpu|).
U32 = 2.0 ** -24
GAMMA_DOT = 64 * U32


def _t(a, device="cpu") -> torch.Tensor:
    """float64 tensor on `device` from a numpy array, a float tensor, or bf16 bits
    (uint16 numpy arrays are bf16 bit patterns, widened exactly)."""
    if isinstance(a, torch.Tensor):
        return a.to(device=device, dtype=torch.float64)
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16).double()
    return torch.from_numpy(a).to(device=device, dtype=torch.float64)


def bf16_ulp(a: torch.Tensor) -> torch.Tensor:
    """Spacing of bf16 numbers (8 significant bits) at |a|, normal range."""
    _, e = torch.frexp(a.abs().clamp_min(2.0 ** -126))  # |a| = m 2^e, 0.5 <= m < 1
    return torch.ldexp(torch.ones_like(a), (e - 8).to(a.dtype))


def out_bound(x, a_gpu, a_ref, out_ref, out_gpu) -> torch.Tensor:
    """Per-element bound on |out_gpu - out_ref|.  x [N][n][D] (values of the
    bf16 sources), alpha [n][N], out [n][D]; float64 tensors."""
    N = x.shape[0]
    ax = x.abs()
    da = (a_gpu - a_ref).abs().T[:, :, None]  # [N][n][1]
    gN = N * U32 / (1 - N * U32)
    b = (da * ax).sum(0) + gN * (a_gpu.abs().T[:, :, None] * ax).sum(0)
    return 0.5 * bf16_ulp(torch.maximum(out_ref.abs(), out_gpu.abs())) + b


U24 = 2.0 ** -16  # relative rounding error of a block sum stored in the 24-bit format


def merged_out_bound(x, a_gpu, a_ref, out_ref, out_gpu, u_rel=0.0) -> torch.Tensor:
    """Per-element bound on |out_gpu - out_ref| for the forward from block sums
    (out' = bf16(fma(a'_p, p, c' U')), c' = exp(m - M) / den): out_bound plus
    the difference between the weight a shared source gets through c' and its
    exponential inside U' and the saved a'_i, which both approximate
    exp(z_i - M) / den.  Each exponential of an argument of size |z_i - M|
    formed in fp32 (one rounding of the argument, scaled by log2 e, then the
    hardware exp2 within a few ulps) is off by at most u (2 |z_i - M| + 4)
    relative, and |z_i - M| = log(max_j a_j / a_i) from the reference
    weights; the shared sum's n fp32 terms and c' U' + a'_p p add (N + 3) u.
    u_rel: the relative error of a stored element of U' (0 for fp32, U24 for
    the 24-bit format), which scales every shared source's part of it.
    Doubled.  x [N][n][D], alpha [n][N]; float64 tensors."""
    N = x.shape[0]
    ar_ = a_ref.T[:, :, None].clamp_min(1e-300)           # [N][n][1]
    spread = torch.log(ar_.max(0, keepdim=True).values / ar_)
    k = U32 * (2 * spread + 4 + N + 3) + u_rel
    k[N - 1] = 0.0                                        # the partial sum's weight is a'_p itself
    extra = (k * a_gpu.abs().T[:, :, None] * x.abs()).sum(0)
    return out_bound(x, a_gpu, a_ref, out_ref, out_gpu) + 2.0 * extra


def sums_bound(x, z) -> torch.Tensor:
    """Per-element bound on |U_gpu - U_ref| for the block sums from the same
    fp32 scores on both sides: each weight exp(z_i - m) formed in fp32 is off
    by at most u (2 |z_i - m| + 4) relative (argument rounding and the
    hardware exp2), and the n-term fp32 sum adds n u of the sum of |terms|;
    doubled.  x [n][T][D], z [L][T][n]; returns [L][T][D]; float64 tensors."""
    n = x.shape[0]
    zm = z - z.max(2, keepdim=True).values                # [L][T][n]
    c = torch.exp(zm) * U32 * (2 * zm.abs() + 4 + n)
    b = torch.zeros((z.shape[0],) + tuple(x.shape[1:]), dtype=x.dtype, device=x.device)
    for i in range(n):
        b += c[:, :, i:i + 1] * x[i].abs()[None]
    return 2.0 * b


def _bwd_coefficients(x, g, w, r_ref, r_gpu, a_ref, a_gpu):
    """The backward's per-token coefficients and bounds on their errors, from
    the reference and the GPU's saved rstd and alpha (their difference covers
    the saved state's own fp32 rounding and underflow)."""
    N, n, D = x.shape
    u = U32
    r = r_ref.T[:, :, None]                   # [N][n][1]
    dr = (r_gpu - r_ref).abs().T[:, :, None]
    a = a_ref.T[:, :, None]
    dal = (a_gpu - a_ref).abs().T[:, :, None]
    gx = x * g[None]
    da = gx.sum(2, keepdim=True)              # g . x_i
    e_da = GAMMA_DOT * gx.abs_().sum(2, keepdim=True)
    del gx
    wxt = x * w[None, None, :]
    wx = wxt.sum(2, keepdim=True)             # w . x_i
    e_wx = GAMMA_DOT * wxt.abs_().sum(2, keepdim=True)
    del wxt
    s = (a * da).sum(0, keepdim=True)
    e_s = (dal * da.abs() + a * e_da + N * u * a * da.abs()).sum(0, keepdim=True)
    dms = (a[None] * (da[:, None] - da[None])).sum(1)  # da_i - s, formed without cancellation
    dz = a * dms
    # the kernels form da_i - s as e_i - sum_j a_j e_j with e_j = da_j - da_m
    # (m: the source of the largest weight), which adds the error of da_m and
    # the roundings of the e_j, at most (N + 2) u max_j |da_j|, to each term
    da_max = da.abs().max(0, keepdim=True).values
    e_m = e_da.max(0, keepdim=True).values + (N + 2) * u * da_max
    e_dz = dal * dms.abs() + a * (e_da + e_s + e_m) + 2 * u * dz.abs()
    c1 = dz * r
    e_c1 = e_dz * r + dz.abs() * dr + u * c1.abs()
    z = r * wx
    e_z = dr * wx.abs() + r * e_wx + u * z.abs()
    k = z * r / D
    e_k = (e_z * r + z.abs() * dr) / D + 2 * u * k.abs()
    return dict(u=u, N=N, n=n, D=D, a=a, dal=dal, c1=c1, e_c1=e_c1, k=k, e_k=e_k)


def dw_bound(x, g, w, r_ref, r_gpu, a_ref, a_gpu) -> torch.Tensor:
    """Per-element bound on |dw_gpu - dw_ref|: dw = sum over tokens and sources
    of c1 x (c1 = dz rstd), each term off by at most e_c1 |x| plus its own
    rounding, and the fp32 sums over the n N terms add n N u sum |c1 x|;
    doubled.  x [N][n][D] and the rest as dsrc_bound; float64 tensors."""
    c = _bwd_coefficients(x, g, w, r_ref, r_gpu, a_ref, a_gpu)
    ax = x.abs()
    cx = (c["c1"].abs() * ax).sum((0, 1))
    b = (c["e_c1"] * ax).sum((0, 1)) + (1 + c["N"] * c["n"]) * c["u"] * cx
    return 2.0 * b


def dsrc_bound(x, g, w, r_ref, r_gpu, a_ref, a_gpu, dsrc_ref, dsrc_gpu, out_bits: int = 16) -> torch.Tensor:
    """Per-element bound on |dsrc_gpu - dsrc_ref| for the overwriting backward.
    x [N][n][D], g [n][D], w [D], r/a [n][N]; float64 tensors.  out_bits: the
    gradient's storage, 16 (bf16: half its ulp) or 32 (fp32: half an fp32
    ulp of the result)."""
    c = _bwd_coefficients(x, g, w, r_ref, r_gpu, a_ref, a_gpu)
    u, a, dal, c1, e_c1, k, e_k = c["u"], c["a"], c["dal"], c["c1"], c["e_c1"], c["k"], c["e_k"]
    # per element: 2 (|da| |g| + u |a g| + e_c1 |inner| + |c1| (e_k |x| + u |inner|) + u (|a g| + |c1 inner|))
    inner = (w[None, None, :] - k * x).abs_()
    b = inner * (e_c1 + 2 * u * c1.abs())
    b += x.abs() * (c1.abs() * e_k)
    b += g.abs()[None] * (dal + 2 * u * a.abs())
    b *= 2.0
    if out_bits == 16:
        b += 0.5 * bf16_ulp(torch.maximum(dsrc_ref.abs(), dsrc_gpu.abs()))
    else:
        b += u * torch.maximum(dsrc_ref.abs(), dsrc_gpu.abs())
    return b


class Accum:
    """Error metrics of a comparison built up over token chunks: relative L2 of
    out and dsrc over everything compared, the largest per-token relative L2,
    the largest alpha and rstd errors, and the largest ratio of an element's
    error to its bound (out_bound / dsrc_bound).  `device` is where the
    comparison arithmetic runs (expected values always come from the oracle
    on the host)."""

    def __init__(self, device="cpu"):
        self.dev = device
        self.sq = {}
        self.mx = {}

    def _add(self, k, v):
        self.sq[k] = self.sq.get(k, 0.0) + float(v)

    def _max(self, k, v):
        self.mx[k] = max(self.mx.get(k, 0.0), float(v))

    def update(self, x, g, w, gpu: dict, ref: dict):
        """x [N][n][D] and g [n][D]: the chunk's inputs (bf16 bits or tensors);
        w [D]; gpu / ref: dicts of out [n][D], rstd and alpha [n][N] and
        optionally dsrc [N][n][D] (tensors or arrays); ref["merged"] true
        when out came from the block sums (merged_out_bound), with
        ref["u_rel"] the relative error of their stored elements."""
        d = self.dev
        go, ro = _t(gpu["out"], d), _t(ref["out"], d)
        ga, ra = _t(gpu["alpha"], d), _t(ref["alpha"], d)
        gr, rr = _t(gpu["rstd"], d), _t(ref["rstd"], d)
        xx = _t(x, d)
        self._max("alpha_max_abs", (ga - ra).abs().max())
        self._max("rstd_max_rel", ((gr - rr).abs() / rr.abs()).max())
        self._add("out_err", (go - ro).square().sum())
        self._add("out_ref", ro.square().sum())
        tok_num = (go - ro).square().sum(1).sqrt()
        tok_den = ro.square().sum(1).sqrt()
        self._max("out_token_rel_l2", (tok_num / torch.where(tok_den > 0, tok_den, torch.ones_like(tok_den))).max())
        if ref.get("merged"):  # the forward from block sums (u_rel: U's storage rounding)
            bo = merged_out_bound(xx, ga, ra, ro, go, ref.get("u_rel", 0.0))
        else:
            bo = out_bound(xx, ga, ra, ro, go)
        self._max("out_elem_ratio", ((go - ro).abs() / bo).max())
        del go, ro
        if "dsrc" in ref:
            gd, rd = _t(gpu["dsrc"], d), _t(ref["dsrc"], d)
            self._add("dsrc_err", (gd - rd).square().sum())
            self._add("dsrc_ref", rd.square().sum())
            tok_num = (gd - rd).square().sum((0, 2)).sqrt()
            tok_den = rd.square().sum((0, 2)).sqrt()
            self._max("dsrc_token_rel_l2",
                      (tok_num / torch.where(tok_den > 0, tok_den, torch.ones_like(tok_den))).max())
            bd = dsrc_bound(xx, _t(g, d), _t(w, d), rr, gr, ra, ga, rd, gd)
            self._max("dsrc_elem_ratio", ((gd - rd).abs() / bd).max())

    def result(self) -> dict:
        e = dict(self.mx)
        e["out_rel_l2"] = (self.sq["out_err"] / max(self.sq["out_ref"], 1e-300)) ** 0.5
        if "dsrc_err" in self.sq:
            e["dsrc_rel_l2"] = (self.sq["dsrc_err"] / max(self.sq["dsrc_ref"], 1e-300)) ** 0.5
        return e


def elementwise_ratios(x_bits, g_bits, w, gpu: dict, ref: dict, device="cpu") -> dict:
    """Largest |gpu - ref| / bound over every element of out (and dsrc when
    present) of the given tokens."""
    acc = Accum(device)
    acc.update(x_bits, g_bits, w, gpu, ref)
    e = acc.result()
    return {k: e[k] for k in ("out_elem_ratio", "dsrc_elem_ratio") if k in e}


def per_token_rel_l2(a, b, token_axis: int) -> float:
    """Largest relative L2 error of any single token's values."""
    a, b = _t(a), _t(b)
    dims = tuple(i for i in range(a.dim()) if i != token_axis)
    num = (a - b).square_().sum(dims).sqrt_()
    den = b.square().sum(dims).sqrt_()
    return float((num / torch.where(den > 0, den, torch.ones_like(den))).max())


def within_tolerance(e: dict) -> bool:
    ok = e["out_rel_l2"] <= TOL_OUT_REL_L2 and e["alpha_max_abs"] <= TOL_ALPHA_ABS and e["rstd_max_rel"] <= TOL_RSTD_REL
    if "dsrc_rel_l2" in e:
        ok = ok and e["dsrc_rel_l2"] <= TOL_DSRC_REL_L2
    if "dw_rel_l2" in e:
        ok = ok and e["dw_rel_l2"] <= TOL_DW_REL_L2
    # element-by-element and per-token checks, where they were computed
    for k in ("out_elem_ratio", "dsrc_elem_ratio"):
        if k in e:
            ok = ok and e[k] <= 1.0
    if "out_token_rel_l2" in e:
        ok = ok and e["out_token_rel_l2"] <= TOL_OUT_REL_L2
    if "dsrc_token_rel_l2" in e:
        ok = ok and e["dsrc_token_rel_l2"] <= TOL_DSRC_REL_L2
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
    return gpu, ref, (src, dout, w)


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

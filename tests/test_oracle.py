"""Pins for the fp64 oracle (CPU only).

The oracle is checked against things other than itself:
  * hand-derived closed forms (tests/golden/hand_derived.json),
  * an independent library route: PyTorch fp64 ``rms_norm`` + ``softmax`` with
    autograd for the backward,
  * central finite differences of the oracle's own forward (pins the backward),
  * invariants of the formula (weights sum to 1, N = 1, w = 0, identical
    sources, permutation, scale invariance at eps = 0, the Euler identity
    sum <dx, x> = sum <out, g> at eps = 0, large scores),
  * bf16-entry vs fp64-entry agreement with torch's own bf16 widening.

``test_pins_catch_planted_mistakes`` compiles mutated copies of the oracle
source (on the CPU, in a temp dir) and asserts every mutant fails some pin.
"""
from __future__ import annotations

import json
from fractions import Fraction
import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "hand_derived.json")
ORACLE_SRC = os.path.join(os.path.dirname(HERE), "oracle", "attnres_oracle.c")

_MATH = {"sqrt": math.sqrt, "exp": math.exp, "log": math.log, "e": math.e, "__builtins__": {}}


def _ev(x):
    if isinstance(x, list):
        return [_ev(v) for v in x]
    return float(eval(x, _MATH)) if isinstance(x, str) else float(x)


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------
# individual pins; each returns a list of failure strings (empty = pass) so the
# mutation test can run them against a broken oracle build
# ----------------------------------------------------------------------------

def pin_golden(orc):
    fails = []
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        D, N, eps = c["D"], c["N"], c["eps"]
        x = np.array(c["x"], dtype=np.float64).reshape(N, 1, D)
        w = np.array(_ev(c["w"]))
        out, rstd, alpha = orc.fwd_f64(x, w, eps)
        exp = c["expect"]
        checks = [("rstd", rstd[0]), ("alpha", alpha[0]), ("out", out[0])]
        if c["g"] is not None:
            g = np.array(c["g"], dtype=np.float64).reshape(1, D)
            dx, dw = orc.bwd_f64(x, w, eps, g)
            checks += [("dx", dx[:, 0, :]), ("dw", dw)]
        for key, got in checks:
            if key not in exp:
                continue
            want = np.array(_ev(exp[key]))
            if not np.allclose(got, want, rtol=1e-12, atol=1e-12):
                fails.append(f"golden {c['name']} {key}: got {got} want {want}")
    return fails


def _torch_route(x, w, eps, g):
    """Independent route: library rms_norm, softmax and autograd in fp64."""
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    D = x.shape[-1]
    xn = torch.nn.functional.rms_norm(xt, (D,), eps=eps)  # [N][T][D]
    z = (xn * wt).sum(-1)  # [N][T]
    a = torch.softmax(z, dim=0)  # over sources
    out = (a.unsqueeze(-1) * xt).sum(0)  # [T][D]
    loss = (out * torch.tensor(g, dtype=torch.float64)).sum()
    loss.backward()
    rstd = torch.rsqrt(xt.detach().pow(2).mean(-1) + eps)
    return (out.detach().numpy(), rstd.T.numpy(), a.detach().T.numpy(), xt.grad.numpy(), wt.grad.numpy())


def _rel(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def pin_torch_route(orc):
    fails = []
    # T = 300 spans several of the oracle's fixed dw chunks
    for seed, (N, T, D, eps) in enumerate([(1, 3, 16, 1e-6), (2, 4, 24, 0.1), (3, 5, 32, 1e-6),
                                          (5, 300, 16, 1e-6), (9, 6, 64, 1e-3), (9, 2, 8, 0.0)]):
        r = _rng(100 + seed)
        x = r.standard_normal((N, T, D)) * (1.0 + np.arange(N))[:, None, None]
        w = r.standard_normal(D) / math.sqrt(D) * 3.0
        g = r.standard_normal((T, D))
        t_out, t_rstd, t_alpha, t_dx, t_dw = _torch_route(x, w, eps, g)
        out, rstd, alpha = orc.fwd_f64(x, w, eps)
        dx, dw = orc.bwd_f64(x, w, eps, g)
        for name, a, b in (("out", out, t_out), ("rstd", rstd, t_rstd), ("alpha", alpha, t_alpha),
                           ("dx", dx, t_dx), ("dw", dw, t_dw)):
            e = _rel(a, b)
            if not e < 1e-11:
                fails.append(f"torch route N={N} T={T} D={D} eps={eps} {name}: rel {e:.3e}")
    return fails


def pin_finite_differences(orc):
    fails = []
    r = _rng(7)
    N, T, D, eps, h = 3, 2, 16, 1e-6, 1e-6
    x = r.standard_normal((N, T, D)) * np.array([1.0, 2.0, 0.5])[:, None, None]
    w = r.standard_normal(D) * 0.5
    g = r.standard_normal((T, D))

    def loss(xx, ww):
        return float((orc.fwd_f64(xx, ww, eps)[0] * g).sum())

    dx, dw = orc.bwd_f64(x, w, eps, g)
    fd_x = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        xp = x.copy()
        xp[idx] += h
        xm = x.copy()
        xm[idx] -= h
        fd_x[idx] = (loss(xp, w) - loss(xm, w)) / (2 * h)
    fd_w = np.zeros_like(w)
    for d in range(D):
        wp = w.copy()
        wp[d] += h
        wm = w.copy()
        wm[d] -= h
        fd_w[d] = (loss(x, wp) - loss(x, wm)) / (2 * h)
    ex, ew = _rel(dx, fd_x), _rel(dw, fd_w)
    if not ex < 1e-6:
        fails.append(f"finite differences dx rel {ex:.3e}")
    if not ew < 1e-6:
        fails.append(f"finite differences dw rel {ew:.3e}")
    return fails


def pin_invariants(orc):
    fails = []
    r = _rng(11)
    N, T, D = 5, 7, 32
    x = r.standard_normal((N, T, D)) * (1.0 + np.arange(N))[:, None, None]
    w = r.standard_normal(D) / math.sqrt(D) * 4.0
    g = r.standard_normal((T, D))
    eps = 1e-6
    out, rstd, alpha = orc.fwd_f64(x, w, eps)
    dx, dw = orc.bwd_f64(x, w, eps, g)
    if not np.allclose(alpha.sum(1), 1.0, atol=1e-14):
        fails.append("alpha does not sum to 1")
    # w = 0: uniform weights, mean of sources, dx_i = g / N
    o0, _, a0 = orc.fwd_f64(x, np.zeros(D), eps)
    dx0, _ = orc.bwd_f64(x, np.zeros(D), eps, g)
    if not (np.allclose(a0, 1.0 / N, atol=1e-15) and np.allclose(o0, x.mean(0), atol=1e-13)
            and np.allclose(dx0, np.broadcast_to(g / N, dx0.shape), atol=1e-13)):
        fails.append("w = 0 invariant")
    # identical sources: out = x, dw = 0, dx_i = alpha_i g
    xi = np.broadcast_to(x[:1], x.shape).copy()
    oi, _, ai = orc.fwd_f64(xi, w, eps)
    dxi, dwi = orc.bwd_f64(xi, w, eps, g)
    if not (np.allclose(oi, x[0], atol=1e-13) and np.allclose(dwi, 0.0, atol=1e-12)
            and np.allclose(dxi, ai.T[:, :, None] * g[None], atol=1e-13)):
        fails.append("identical-sources invariant")
    # permutation of the sources
    p = np.array([3, 0, 4, 1, 2])
    op, _, ap = orc.fwd_f64(x[p], w, eps)
    dxp, dwp = orc.bwd_f64(x[p], w, eps, g)
    if not (np.allclose(op, out, atol=1e-12) and np.allclose(ap, alpha[:, p], atol=1e-14)
            and np.allclose(dxp, dx[p], atol=1e-12) and np.allclose(dwp, dw, atol=1e-11)):
        fails.append("permutation invariant")
    # eps = 0: scaling a source leaves its weight unchanged; scaling all scales out
    o_e0, _, a_e0 = orc.fwd_f64(x, w, 0.0)
    xs = x.copy()
    xs[2] *= 37.0
    _, _, a_s = orc.fwd_f64(xs, w, 0.0)
    o_all, _, a_all = orc.fwd_f64(x * 0.125, w, 0.0)
    if not (np.allclose(a_s, a_e0, atol=1e-14) and np.allclose(a_all, a_e0, atol=1e-14)
            and np.allclose(o_all, 0.125 * o_e0, atol=1e-13)):
        fails.append("scale invariance at eps = 0")
    # eps = 0: out is 1-homogeneous in x, so sum <dx, x> = sum <out, g>
    dx_e0, _ = orc.bwd_f64(x, w, 0.0, g)
    lhs, rhs = float((dx_e0 * x).sum()), float((o_e0 * g).sum())
    if not abs(lhs - rhs) <= 1e-10 * max(1.0, abs(rhs)):
        fails.append(f"Euler identity {lhs} vs {rhs}")
    # token independence: a token's result does not depend on the other tokens
    o_sub, r_sub, a_sub = orc.fwd_f64(x[:, 2:5], w, eps)
    dx_sub, _ = orc.bwd_f64(x[:, 2:5], w, eps, g[2:5])
    if not (np.array_equal(o_sub, out[2:5]) and np.array_equal(a_sub, alpha[2:5])
            and np.array_equal(r_sub, rstd[2:5]) and np.array_equal(dx_sub, dx[:, 2:5])):
        fails.append("token independence")
    # large scores (|z| ~ 1e3): weights stay finite and sum to 1
    wl = w * 400.0
    ol, _, al = orc.fwd_f64(x, wl, eps)
    if not (np.isfinite(al).all() and np.isfinite(ol).all() and np.allclose(al.sum(1), 1.0, atol=1e-14)):
        fails.append("large-score softmax not finite")
    # N = 2 closed form: alpha_0 = sigmoid(z_0 - z_1), with z from torch's rms_norm
    x2 = x[:2]
    _, _, a2 = orc.fwd_f64(x2, w, eps)
    z = (torch.nn.functional.rms_norm(torch.tensor(x2), (D,), eps=eps) * torch.tensor(w)).sum(-1).numpy()
    if not np.allclose(a2[:, 0], 1.0 / (1.0 + np.exp(-(z[0] - z[1]))), atol=1e-14):
        fails.append("N = 2 sigmoid closed form")
    return fails


def pin_bf16_entry(orc):
    """The bf16 entry points widen exactly: compare with torch's own bf16 -> fp64."""
    fails = []
    wl = synth.Workload("pin", T=260, N=4, D=64, kind="depth")
    src = wl.sources()
    dout = wl.dout()
    w = wl.w()
    xs = torch.from_numpy(src.view(np.int16)).view(torch.bfloat16).double().numpy()
    gs = torch.from_numpy(dout.view(np.int16)).view(torch.bfloat16).double().numpy()
    out, rstd, alpha = orc.fwd(src, w, wl.eps)
    dsrc, dw = orc.bwd(src, w, wl.eps, dout)
    out2, rstd2, alpha2 = orc.fwd_f64(xs, w.astype(np.float64), float(np.float32(wl.eps)))
    dx2, dw2 = orc.bwd_f64(xs, w.astype(np.float64), float(np.float32(wl.eps)), gs)
    for name, a, b in (("out", out, out2), ("rstd", rstd, rstd2), ("alpha", alpha, alpha2),
                       ("dsrc", dsrc, dx2), ("dw", dw, dw2)):
        if not np.allclose(a, b, rtol=1e-13, atol=1e-13):
            fails.append(f"bf16 entry {name} differs from fp64 entry")
    _, dw_only = orc.bwd(src, w, wl.eps, dout, want_dsrc=False)
    if not np.array_equal(dw_only, dw):
        fails.append("dw-only backward differs")
    return fails


ROUNDING_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "partial_sum_rounding.json")


def _bf16_value(bits: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern (sign, 8-bit exponent, 7-bit fraction)."""
    sign = -1 if bits & 0x8000 else 1
    e, f = (bits >> 7) & 0xFF, bits & 0x7F
    if e == 0:
        return sign * Fraction(f, 1 << 7) * Fraction(1, 1 << 126)
    return sign * (1 + Fraction(f, 1 << 7)) * (Fraction(2) ** (e - 127))


def _round_to_bf16(v: Fraction, negative_zero: bool = False) -> int:
    """Nearest bf16 to the exact rational v, ties to even, by exhaustive
    comparison with the two neighbouring bf16 values (independent of the C
    oracle's frexp/nearbyint route)."""
    if v == 0:
        return 0x8000 if negative_zero else 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    if a >= (2 - Fraction(1, 1 << 8)) * (Fraction(2) ** 127):
        return sign | 0x7F80
    lo, hi = 0, 0x7F7F  # positive finite patterns are ordered like their values
    while lo < hi:  # largest pattern whose value is <= a
        mid = (lo + hi + 1) // 2
        if _bf16_value(mid) <= a:
            lo = mid
        else:
            hi = mid - 1
    below, above = lo, lo + 1
    if _bf16_value(below) == a:
        return sign | below
    d_lo, d_hi = a - _bf16_value(below), _bf16_value(above) - a
    if d_lo < d_hi or (d_lo == d_hi and below % 2 == 0):
        return sign | below
    return sign | above


def pin_partial_sum_update(orc):
    """bf16(p + y): hand-worked rounding cases, then exact rational arithmetic
    on random pairs concentrated on near ties and close exponents."""
    fails = []
    cases = json.load(open(ROUNDING_GOLDEN))["cases"]
    p = np.array([int(c["p"], 16) for c in cases], dtype=np.uint16)
    y = np.array([int(c["y"], 16) for c in cases], dtype=np.uint16)
    got = orc.add_bf16(p, y)
    for c, g in zip(cases, got):
        if int(g) != int(c["expect"], 16):
            fails.append(f"rounding golden {c['name']}: got {int(g):04X} want {c['expect']}")
    rng = np.random.default_rng(11)
    n = 4000
    # exponents within a few binades of each other (where ties happen), plus spread-out ones
    e1 = rng.integers(100, 150, n)
    e2 = np.where(rng.random(n) < 0.7, e1 - rng.integers(0, 10, n), rng.integers(1, 254, n))
    pb = ((rng.integers(0, 2, n) << 15) | (e1 << 7) | rng.integers(0, 128, n)).astype(np.uint16)
    yb = ((rng.integers(0, 2, n) << 15) | (np.clip(e2, 1, 254) << 7) | rng.integers(0, 128, n)).astype(np.uint16)
    got = orc.add_bf16(pb, yb)
    for a, b, g in zip(pb.tolist(), yb.tolist(), got.tolist()):
        want = _round_to_bf16(_bf16_value(a) + _bf16_value(b), negative_zero=bool(a & b & 0x8000))
        if g != want:
            fails.append(f"rounding {a:04X}+{b:04X}: got {g:04X} want {want:04X}")
            if len(fails) > 5:
                break
    # the fused forward's last source is the updated partial sum
    src = rng.integers(0x3E00, 0x4100, (2, 3, 16)).astype(np.uint16)
    pp = rng.integers(0x3E00, 0x4100, (3, 16)).astype(np.uint16)
    yy = rng.integers(0x3C00, 0x3F00, (3, 16)).astype(np.uint16)
    w = rng.standard_normal(16).astype(np.float32)
    out, _, alpha, p_new = orc.fwd_update(src, pp, yy, w, 1e-6)
    ref_out, _, ref_alpha = orc.fwd(np.concatenate([src, orc.add_bf16(pp, yy)[None]]), w, 1e-6)
    if not (np.array_equal(out, ref_out) and np.array_equal(alpha, ref_alpha)):
        fails.append("fwd_update does not use bf16(p + y) as the last source")
    return fails


GOLDEN_BLOCK = os.path.join(HERE, "golden", "block_scores.json")


def _bits_of(values) -> np.ndarray:
    """bf16 bit patterns of values that are exact in bf16."""
    f = np.asarray(values, dtype=np.float32)
    b = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((b.astype(np.uint32) << 16).view(np.float32), f), "not exact in bf16"
    return b


def _random_bits(r, shape, scales):
    """Random bf16 bit patterns, source i scaled by scales[i] (rounded to bf16 by truncation of the draw)."""
    x = (r.standard_normal(shape) * np.asarray(scales)[:, None, None]).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def pin_block_scores(orc):
    """Block-batched scores: hand-derived constant-row cases; PyTorch fp64
    rms_norm + matmul (library route); the softmax of each sub-layer's scores
    equals the plain forward's weights for that sub-layer's pseudo-query."""
    fails = []
    for c in json.load(open(GOLDEN_BLOCK))["block_scores"]:
        x = _bits_of(c["x"])[:, None, :]  # [n][1][D]
        W = np.array(c["W"], dtype=np.float32)
        rstd, z = orc.block_scores(x, W, c["eps"])
        want_r = np.array(_ev(c["expect"]["rstd"]))
        want_z = np.array(_ev(c["expect"]["z"]))  # [L][n]
        if not np.allclose(rstd[0], want_r, rtol=1e-12, atol=1e-12):
            fails.append(f"block golden {c['name']} rstd: {rstd[0]} vs {want_r}")
        if not np.allclose(z[:, 0, :], want_z, rtol=1e-12, atol=1e-12):
            fails.append(f"block golden {c['name']} z: {z[:, 0, :]} vs {want_z}")
    for seed, (n, T, D, L, eps) in enumerate([(1, 3, 16, 2, 1e-6), (3, 5, 32, 4, 0.1), (8, 7, 64, 24, 1e-6),
                                             (2, 4, 8, 3, 0.0)]):
        r = _rng(300 + seed)
        bits = _random_bits(r, (n, T, D), 1.0 + np.arange(n))
        W = (r.standard_normal((L, D)) / math.sqrt(D) * 2.0).astype(np.float32)
        rstd, z = orc.block_scores(bits, W, eps)
        xt = torch.from_numpy(oracle.bf16_to_f64(bits))
        xn = torch.nn.functional.rms_norm(xt, (D,), eps=eps)                 # [n][T][D]
        z_t = torch.matmul(xn, torch.from_numpy(W.astype(np.float64)).T)     # [n][T][L]
        r_t = (xn * xt).sum(-1) / (xt * xt).sum(-1)                          # the factor rms_norm applied
        e_z = _rel(z, z_t.permute(2, 1, 0).numpy())
        e_r = _rel(rstd, r_t.T.numpy())
        if not (e_z < 1e-12 and e_r < 1e-12):
            fails.append(f"block torch route n={n} T={T} D={D} L={L}: z rel {e_z:.3e}, rstd rel {e_r:.3e}")
        for l in range(L):
            _, _, a_plain = orc.fwd(bits, W[l], eps)
            zz = z[l] - z[l].max(axis=1, keepdims=True)
            a_blk = np.exp(zz) / np.exp(zz).sum(axis=1, keepdims=True)
            if not np.allclose(a_blk, a_plain, rtol=1e-12, atol=1e-14):
                fails.append(f"block scores of sub-layer {l} do not give the plain forward's weights")
                break
    return fails


def pin_fwd_scored(orc):
    """Forward from given scores: the two-source closed form with a given score;
    with the scores and rstd of the first N-1 sources from block_scores, every
    output equals the plain forward on all N sources."""
    fails = []
    for c in json.load(open(GOLDEN_BLOCK))["fwd_scored"]:
        x = _bits_of(c["x"])[:, None, :]
        zg = np.array(_ev(c["z_given"]))[None, :]
        rg = np.array(_ev(c["r_given"]))[None, :]
        out, rstd, alpha = orc.fwd_scored(x, zg, rg, np.array(c["w"], dtype=np.float32), c["eps"])
        for key, got in (("alpha", alpha[0]), ("out", out[0]), ("rstd", rstd[0])):
            want = np.array(_ev(c["expect"][key]))
            if not np.allclose(got, want, rtol=1e-12, atol=1e-12):
                fails.append(f"scored golden {c['name']} {key}: {got} vs {want}")
    for seed, (N, T, D, eps) in enumerate([(2, 3, 16, 1e-6), (5, 6, 32, 0.05), (9, 9, 64, 1e-6), (9, 4, 8, 0.0)]):
        r = _rng(400 + seed)
        bits = _random_bits(r, (N, T, D), np.sqrt(1.0 + 12.0 * np.arange(N)))
        W = (r.standard_normal((3, D)) * 0.5).astype(np.float32)
        rb, zb = orc.block_scores(bits[:N - 1], W, eps)
        for l in range(3):
            got = orc.fwd_scored(bits, zb[l], rb, W[l], eps)
            want = orc.fwd(bits, W[l], eps)
            for name, a, b in zip(("out", "rstd", "alpha"), got, want):
                e = _rel(a, b)
                if not e < 1e-12:
                    fails.append(f"scored vs plain N={N} T={T} D={D} l={l} {name}: rel {e:.3e}")
    return fails


def pin_block_sums(orc):
    """Block-batched shared sums: hand-worked sums; one shared source gives the
    source itself exactly; adding a constant to a sub-layer's scores leaves its
    sum unchanged; each sum divided by its weights' total is the plain forward
    on the shared sources alone for that sub-layer's pseudo-query."""
    fails = []
    for c in json.load(open(GOLDEN_BLOCK))["block_sums"]:
        x = _bits_of(c["x"])[:, None, :]                      # [n][1][D]
        z = np.array(_ev(c["z"]))[:, None, :]                 # [L][1][n]
        U = orc.block_sums(x, z)
        want = np.array(_ev(c["expect"]))                     # [L][D]
        if not np.allclose(U[:, 0, :], want, rtol=1e-13, atol=1e-13):
            fails.append(f"sums golden {c['name']}: {U[:, 0, :]} vs {want}")
    r = _rng(500)
    bits = _random_bits(r, (1, 5, 24), [3.0])
    z1 = r.standard_normal((4, 5, 1)) * 7.0
    if not np.array_equal(orc.block_sums(bits, z1), np.broadcast_to(oracle.bf16_to_f64(bits), (4, 5, 24))):
        fails.append("one shared source: the sum is not the source itself")
    for seed, (n, T, D, L, eps) in enumerate([(2, 3, 16, 2, 1e-6), (5, 6, 32, 4, 0.05), (8, 7, 64, 24, 1e-6)]):
        r = _rng(510 + seed)
        bits = _random_bits(r, (n, T, D), np.sqrt(1.0 + 12.0 * np.arange(n)))
        W = (r.standard_normal((L, D)) * 0.5).astype(np.float32)
        rb, zb = orc.block_scores(bits, W, eps)
        U = orc.block_sums(bits, zb)
        e = _rel(orc.block_sums(bits, zb + 3.75), U)
        if not e < 1e-13:
            fails.append(f"sums not shift invariant n={n}: rel {e:.3e}")
        tot = np.exp(zb - zb.max(axis=2, keepdims=True)).sum(axis=2)  # [L][T]
        for l in range(L):
            out, _, _ = orc.fwd(bits, W[l], eps)
            e = _rel(U[l] / tot[l][:, None], out)
            if not e < 1e-12:
                fails.append(f"sums / weights vs plain forward on the shared sources n={n} l={l}: rel {e:.3e}")
                break
    return fails


def pin_fwd_merged(orc):
    """Forward from the shared sum: hand-worked cases with the given or the
    partial sum's score the largest; through block_scores and block_sums it
    reproduces the plain forward on all N sources; shared scores far below the
    partial sum's give out = p and alpha = (0, .., 0, 1) exactly, far above it
    the shared sums normalised by their own weights."""
    fails = []
    for c in json.load(open(GOLDEN_BLOCK))["fwd_merged"]:
        U = np.array(_ev(c["U"]))[None, :]
        p = _bits_of(c["p"])[None, :]
        zg = np.array(_ev(c["z_given"]))[None, :]
        rg = np.array(_ev(c["r_given"]))[None, :]
        out, rstd, alpha = orc.fwd_merged(U, p, zg, rg, np.array(c["w"], dtype=np.float32), c["eps"])
        for key, got in (("alpha", alpha[0]), ("out", out[0]), ("rstd", rstd[0])):
            want = np.array(_ev(c["expect"][key]))
            if not np.allclose(got, want, rtol=1e-12, atol=1e-12):
                fails.append(f"merged golden {c['name']} {key}: {got} vs {want}")
    for seed, (N, T, D, eps, wstd) in enumerate([(2, 3, 16, 1e-6, 0.5), (5, 6, 32, 0.05, 0.5), (9, 9, 64, 1e-6, 0.5),
                                                (9, 5, 32, 0.0, 4.0)]):
        r = _rng(520 + seed)
        bits = _random_bits(r, (N, T, D), np.sqrt(1.0 + 12.0 * np.arange(N)))
        W = (r.standard_normal((3, D)) * wstd).astype(np.float32)
        rb, zb = orc.block_scores(bits[:N - 1], W, eps)
        U = orc.block_sums(bits[:N - 1], zb)
        for l in range(3):
            got = orc.fwd_merged(U[l], bits[N - 1], zb[l], rb, W[l], eps)
            want = orc.fwd(bits, W[l], eps)
            for name, a, b in zip(("out", "rstd", "alpha"), got, want):
                e = _rel(a, b)
                if not e < 1e-12:
                    fails.append(f"merged vs plain N={N} T={T} D={D} l={l} {name}: rel {e:.3e}")
    r = _rng(530)
    N, T, D = 4, 3, 16
    bits = _random_bits(r, (N, T, D), [1.0, 2.0, 3.0, 4.0])
    w = (r.standard_normal(D) * 0.1).astype(np.float32)
    rg = np.ones((T, N - 1))
    U = r.standard_normal((T, D))
    out, _, alpha = orc.fwd_merged(U, bits[N - 1], np.full((T, N - 1), -1000.0), rg, w, 1e-6)
    if not (np.array_equal(out, oracle.bf16_to_f64(bits[N - 1])) and np.array_equal(alpha[:, N - 1], np.ones(T))
            and not alpha[:, :N - 1].any()):
        fails.append("shared scores far below the partial sum's: out is not p")
    zg = 1000.0 + r.standard_normal((T, N - 1))
    out, _, _ = orc.fwd_merged(U, bits[N - 1], zg, rg, w, 1e-6)
    want = U / np.exp(zg - zg.max(axis=1, keepdims=True)).sum(axis=1, keepdims=True)
    if not np.allclose(out, want, rtol=1e-13, atol=1e-13):
        fails.append("shared scores far above the partial sum's: out is not the normalised shared sum")
    return fails


def pin_softmax_bwd_one_hot(orc):
    """A token whose weights are one-hot to within fp64 rounding.  Two sources,
    D = 2, eps = 0: x_0 = (1, 0), x_1 = (0, 2) normalise to (sqrt 2, 0) and
    (0, sqrt 2); with w = (0, 100 / sqrt 2) the scores are 0 and 100, so
    alpha_0 = 1 / (1 + e^100) (3.7e-44) and alpha_1 = 1 - alpha_0 (1.0 in
    fp64).  With g = (3, 1), da = (3, 2), and the softmax Jacobian gives
    dz_0 = alpha_0 alpha_1 (da_0 - da_1) = -dz_1, so
    dw = sum_i dz_i r_i x_i = sqrt 2 alpha_0 alpha_1 (1, -1): the dominant
    source's dz must not vanish although da_1 - s is far below da_1's
    rounding."""
    fails = []
    x = np.array([[[1.0, 0.0]], [[0.0, 2.0]]])
    w = np.array([0.0, 100.0 / math.sqrt(2.0)])
    g = np.array([[3.0, 1.0]])
    _, _, alpha = orc.fwd_f64(x, w, 0.0)
    _, dw = orc.bwd_f64(x, w, 0.0, g)
    a0 = 1.0 / (1.0 + math.exp(100.0))
    want = math.sqrt(2.0) * a0 * (1.0 - a0) * np.array([1.0, -1.0])
    if not (abs(alpha[0, 0] - a0) <= 1e-12 * a0 and alpha[0, 1] == 1.0):
        fails.append(f"one-hot weights: {alpha}")
    if not np.allclose(dw, want, rtol=1e-12, atol=0.0):
        fails.append(f"one-hot softmax backward: dw {dw} want {want}")
    return fails


U24_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "u24_format.json")


def _f32_value(bits: int) -> Fraction:
    """Exact value of a finite binary32 bit pattern."""
    sign = -1 if bits & 0x80000000 else 1
    e, f = (bits >> 23) & 0xFF, bits & 0x7FFFFF
    if e == 0:
        return sign * Fraction(f, 1 << 23) * Fraction(1, 1 << 126)
    return sign * (1 + Fraction(f, 1 << 23)) * (Fraction(2) ** (e - 127))


def _round16(v: Fraction):
    """v rounded to 16 significant bits, nearest, ties to even, with the
    quantum 2^-141 below 2^-126; None where it reaches 2^128 (infinity).
    Worked on exact rationals from the rule, independently of the C route."""
    a = abs(v)
    if a == 0:
        return Fraction(0)
    e = a.numerator.bit_length() - a.denominator.bit_length()  # 2^e <= a < 2^(e+2)
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    while Fraction(2) ** e > a:
        e -= 1
    quantum = Fraction(2) ** (max(e, -126) - 15)
    n = a / quantum
    lo = n.numerator // n.denominator
    rem = n - lo
    k = lo + 1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1) else lo
    r = k * quantum
    if r >= Fraction(2) ** 128:
        return None
    return r if v > 0 else -r


def pin_u24_format(orc):
    """The shared sums' 24-bit storage format: hand-worked encodings and
    decodings, then exact rational rounding of random binary32 values
    concentrated on ties, and exactness on values that already fit."""
    fails = []
    g = json.load(open(U24_GOLDEN))
    xs = np.array([int(c["x"], 16) for c in g["round"]], dtype=np.uint32).view(np.float32)
    got = orc.round24(xs)
    for c, b in zip(g["round"], got):
        if bytes(b.tolist()).hex().upper() != c["expect"]:
            fails.append(f"u24 golden {c['name']}: got {bytes(b.tolist()).hex()} want {c['expect']}")
    bs = np.array([list(bytes.fromhex(c["bytes"])) for c in g["decode"]], dtype=np.uint8)
    dec = orc.decode24(bs).view(np.uint32)
    for c, d in zip(g["decode"], dec.tolist()):
        if d != int(c["expect"], 16):
            fails.append(f"u24 decode golden {c['name']}: got {d:08X} want {c['expect']}")
    rng = np.random.default_rng(23)
    n = 3000
    e = np.where(rng.random(n) < 0.1, rng.integers(0, 3, n), rng.integers(1, 255, n)).astype(np.uint32)
    low = rng.choice(np.array([0x7F, 0x80, 0x81, 0x00, 0xFF], dtype=np.uint32), n)
    low = np.where(rng.random(n) < 0.3, rng.integers(0, 256, n).astype(np.uint32), low)
    pat = (rng.integers(0, 2, n).astype(np.uint32) << 31) | (e << 23) | (rng.integers(0, 1 << 15, n).astype(np.uint32) << 8) | low
    x = pat.view(np.float32)
    back = orc.decode24(orc.round24(x)).view(np.uint32)
    for p_, b_ in zip(pat.tolist(), back.tolist()):
        r = _round16(_f32_value(p_))
        want = (0x7F800000 | (p_ & 0x80000000)) if r is None else None
        if want is None:
            want = int(np.array([float(r)], dtype=np.float32).view(np.uint32)[0])  # r has <= 16 bits: exact
            if r == 0 and p_ & 0x80000000:
                want = 0x80000000
        if b_ != want:
            fails.append(f"u24 rounding of {p_:08X}: got {b_:08X} want {want:08X}")
            if len(fails) > 10:
                break
    fit = (pat & np.uint32(0xFFFFFF00)) & np.uint32(0xFF7FFFFF)  # zero low byte, finite exponents
    if not np.array_equal(orc.decode24(orc.round24(fit.view(np.float32))).view(np.uint32), fit):
        fails.append("u24: a value with 16 significant bits did not survive the round trip")
    return fails


PINS = [pin_golden, pin_torch_route, pin_finite_differences, pin_invariants, pin_bf16_entry, pin_partial_sum_update,
        pin_block_scores, pin_fwd_scored, pin_block_sums, pin_fwd_merged, pin_u24_format, pin_softmax_bwd_one_hot]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    fails = pin(oracle.default())
    assert not fails, "\n".join(fails)


# ----------------------------------------------------------------------------
# planted mistakes: each mutant of the oracle source must fail at least one pin
# ----------------------------------------------------------------------------

MUTANTS = {
    "sum_not_mean": ("r[i] = 1.0 / sqrt(ss / (double)D + eps);", "r[i] = 1.0 / sqrt(ss + eps);"),
    "eps_outside_sqrt": ("r[i] = 1.0 / sqrt(ss / (double)D + eps);", "r[i] = 1.0 / sqrt(ss / (double)D) + eps;"),
    "eps_dropped": ("r[i] = 1.0 / sqrt(ss / (double)D + eps);", "r[i] = 1.0 / sqrt(ss / (double)D);"),
    "score_unnormalised": ("dot += w[d] * (r[i] * x[i][d]);", "dot += w[d] * x[i][d];"),
    "no_max_subtraction": ("alpha[i] = exp(z[i] - m) / den;", "alpha[i] = exp(z[i]) / den * exp(-m);"),
    "values_normalised": ("acc += alpha[i] * x[i][d];", "acc += alpha[i] * r[i] * x[i][d];"),
    "softmax_bwd_sign": ("acc += alpha[j] * (da[i] - da[j]);", "acc += alpha[j] * (da[j] - da[i]);"),
    "direct_term_dropped": ("dx[i][d] = alpha[i] * g[d] + dz[i]", "dx[i][d] = dz[i]"),
    "rstd_term_dropped": ("(w[d] - z[i] * r[i] * x[i][d] / (double)D)", "(w[d])"),
    "dw_missing_rstd": ("dw[d] += dz[i] * r[i] * x[i][d];", "dw[d] += dz[i] * x[i][d];"),
    "da_uses_w": ("acc += g[d] * x[i][d];", "acc += w[d] * x[i][d];"),
    "token_major_rows": ("rows[i] = x + ((int64_t)i * T + t) * D;", "rows[i] = x + (t * N + i) * D;"),
    "alpha_transposed": ("if (alpha) alpha[t * N + i] = a[i];", "if (alpha) alpha[i * T + t] = a[i];"),
    "dw_chunks_overwrite": ("dw[d] += part[c * D + d];", "dw[d] = part[c * D + d];"),
    "bf16_widen_shift": ("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    "w_narrowed": ("wd[d] = (double)w[d];", "wd[d] = (double)(int)(w[d] * 64.0) / 64.0;"),
    "update_truncates": ("nearbyint(ldexp(m, keep))", "floor(ldexp(m, keep))"),
    "update_ties_away": ("nearbyint(ldexp(m, keep))", "round(ldexp(m, keep))"),
    "update_nine_bits": ("int keep = 8;", "int keep = 9;"),
    "update_drops_output": ("bf16_to_f64(p[k]) + bf16_to_f64(y[k])", "bf16_to_f64(p[k])"),
    "softmax_den_skips_first": ("for (int i = 0; i < N; ++i) den += exp(z[i] - m);",
                                "for (int i = 1; i < N; ++i) den += exp(z[i] - m);"),
    "weighted_sum_skips_first": ("for (int i = 0; i < N; ++i) acc += alpha[i] * x[i][d];",
                                 "for (int i = 1; i < N; ++i) acc += alpha[i] * x[i][d];"),
    "softmax_bwd_unweighted_mean": ("acc += alpha[j] * (da[i] - da[j]);", "acc += (da[i] - da[j]) / N;"),
    "softmax_jacobian_first_form": ("for (int j = 0; j < N; ++j) acc += alpha[j] * (da[i] - da[j]);\n    dz[i] = alpha[i] * acc;",
                                    "for (int j = 0; j < N; ++j) acc += alpha[j] * da[j];\n    dz[i] = alpha[i] * (da[i] - acc);"),
    "mean_abs_not_square": ("for (int64_t d = 0; d < D; ++d) ss += x[i][d] * x[i][d];",
                            "for (int64_t d = 0; d < D; ++d) ss += fabs(x[i][d]);"),
    "dw_drops_last_chunk": ("for (int64_t c = 0; c < nchunk; ++c)\n    for (int64_t d = 0; d < D; ++d) dw[d] += part",
                            "for (int64_t c = 0; c + 1 < nchunk; ++c)\n    for (int64_t d = 0; d < D; ++d) dw[d] += part"),
    "dout_of_token_zero": ("g[d] = bf16_to_f64(dout[t * D + d]);", "g[d] = bf16_to_f64(dout[d]);"),
    # block-batched scores and the forward from given scores
    "block_sum_not_mean": ("const double rb = 1.0 / sqrt(sq / (double)D + eps);",
                           "const double rb = 1.0 / sqrt(sq + eps);"),
    "block_eps_outside_sqrt": ("const double rb = 1.0 / sqrt(sq / (double)D + eps);",
                               "const double rb = 1.0 / sqrt(sq / (double)D) + eps;"),
    "block_W_transposed": ("acc += (double)W[(int64_t)l * D + d] * (rb * bf16_to_f64(row[d]));",
                           "acc += (double)W[d * L + l] * (rb * bf16_to_f64(row[d]));"),
    "block_score_unnormalised": ("acc += (double)W[(int64_t)l * D + d] * (rb * bf16_to_f64(row[d]));",
                                 "acc += (double)W[(int64_t)l * D + d] * bf16_to_f64(row[d]);"),
    "block_z_token_major": ("z[((int64_t)l * T + t) * n + i] = acc;", "z[((int64_t)t * L + l) * n + i] = acc;"),
    "scored_first_score_everywhere": ("zs[i] = zg[t * (N - 1) + i];", "zs[i] = zg[t * (N - 1)];"),
    "scored_rstd_not_given": ("rs[i] = rg[t * (N - 1) + i];", "rs[i] = 1.0;"),
    "scored_last_unnormalised": ("acc += (double)w[d] * (rs[N - 1] * bf16_to_f64(last[d]));",
                                 "acc += (double)w[d] * bf16_to_f64(last[d]);"),
    "scored_last_is_first_source": ("const uint16_t* last = src + ((int64_t)(N - 1) * T + t) * D;",
                                    "const uint16_t* last = src + t * D;"),
    "scored_sum_skips_last": ("for (int i = 0; i < N; ++i) o += as[i]", "for (int i = 0; i + 1 < N; ++i) o += as[i]"),
    # block-batched shared sums and the forward from them
    "sums_no_max_subtraction": ("acc += exp(zt[i] - m) * bf16_to_f64", "acc += exp(zt[i]) * bf16_to_f64"),
    "sums_skip_first_source": ("for (int i = 0; i < n; ++i) acc += exp(zt[i] - m)",
                               "for (int i = 1; i < n; ++i) acc += exp(zt[i] - m)"),
    "sums_max_of_first_score": ("for (int i = 1; i < n; ++i)\n        if (zt[i] > m) m = zt[i];", ""),
    "sums_z_token_major": ("const double* zt = z + ((int64_t)l * T + t) * n;",
                           "const double* zt = z + ((int64_t)t * L + l) * n;"),
    "sums_normalised_rows": ("acc += exp(zt[i] - m) * bf16_to_f64(src[((int64_t)i * T + t) * D + d]);",
                             "acc += exp(zt[i] - m) * bf16_to_f64(src[((int64_t)i * T + t) * D + d]) / (1.0 + i);"),
    "merged_no_rescale": ("const double shared = exp(m - top)", "const double shared = 1.0"),
    "merged_den_skips_partial": ("for (int i = 0; i < N; ++i) den += exp(zs[i] - top);",
                                 "for (int i = 0; i + 1 < N; ++i) den += exp(zs[i] - top);"),
    "merged_partial_unweighted": ("own * bf16_to_f64(pt[d])", "bf16_to_f64(pt[d])"),
    "merged_partial_unnormalised": ("dot += (double)w[d] * (rs[N - 1] * bf16_to_f64(pt[d]));",
                                    "dot += (double)w[d] * bf16_to_f64(pt[d]);"),
    "merged_alpha_shifted_by_given_max": ("alpha[t * N + i] = exp(zs[i] - top) / den;",
                                          "alpha[t * N + i] = exp(zs[i] - m) / den;"),
    "merged_shared_of_token_zero": ("shared * U[t * D + d]", "shared * U[d]"),
    # the shared sums' 24-bit storage format
    "u24_truncates": ("r = ldexp(nearbyint(ldexp(m, keep)), e - keep);", "r = ldexp(floor(ldexp(m, keep)), e - keep);"),
    "u24_ties_away": ("r = ldexp(nearbyint(ldexp(m, keep)), e - keep);", "r = ldexp(round(ldexp(m, keep)), e - keep);"),
    "u24_fifteen_bits": ("int keep = 16;", "int keep = 15;"),
    "u24_no_subnormal_quantum": ("        if (e - 1 < -126) keep -= -126 - (e - 1);\n        r = ldexp",
                                 "        r = ldexp"),
    "u24_top_byte_wrong": ("out[3 * k + 2] = (uint8_t)(u >> 24);", "out[3 * k + 2] = (uint8_t)(u >> 16);"),
    "u24_sign_dropped": ("f = (float)(signbit(v) ? -r : r);", "f = (float)r;"),
    "u24_decode_shifted": ("((uint32_t)in[3 * k] << 8)", "((uint32_t)in[3 * k] << 0)"),
}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name, mutant_dir):
    old, new = MUTANTS[name]
    src = open(ORACLE_SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found in the oracle source"
    mutated = src.replace(old, new)
    c_path = os.path.join(mutant_dir, f"{name}.c")
    so_path = os.path.join(mutant_dir, f"{name}.so")
    with open(c_path, "w") as f:
        f.write(mutated)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-o", so_path, c_path, "-lm"],
                   check=True)
    orc = oracle.Oracle(so_path)
    caught = []
    for pin in PINS:
        with np.errstate(all="ignore"):
            if pin(orc):
                caught.append(pin.__name__)
    assert caught, f"planted mistake {name} passed every pin"

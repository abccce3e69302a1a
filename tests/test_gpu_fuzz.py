"""Seeded random configurations through every call, against the fp64 oracle.

Each case draws N, T, D, eps, the source scales, a layout (stacked, separate
buffers, interleaved by token, padded rows) and a call mix (overwriting or
accumulating backward with bf16 or fp32 gradients, decoding forward, fused
partial-sum update), runs it
on the GPU and compares every output with the oracle at the operator's
tolerances.  A second set of cases runs the block-level route (block scores,
block sums, merged forwards) the same way.  The cases are fixed by their seeds, so a failure names a
reproducible configuration."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_residuals_depth_amd as ar
import oracle
import synth
from parity import (DEV, TOL_ALPHA_ABS, TOL_DSRC_REL_L2, TOL_DW_REL_L2, TOL_OUT_REL_L2, TOL_RSTD_REL, U32, _t,
                    bf16_dev_to_f64, dsrc_bound, dw_bound, rel_l2, to_dev_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ar.library()


def _place(src: torch.Tensor, layout: str, rng):
    """Views of the N sources [T][D] in the given layout (the data is the same)."""
    N, T, D = src.shape
    if layout == "separate":
        return [src[i].clone() for i in range(N)]
    if layout == "interleaved":
        cache = src.permute(1, 0, 2).contiguous()
        return [cache[:, i] for i in range(N)]
    pad = 8 * int(rng.integers(1, 20))  # padded rows: pitch D + pad
    buf = torch.zeros((N, T, D + pad), dtype=src.dtype, device=src.device)
    buf[:, :, :D] = src
    return [buf[i, :, :D] for i in range(N)]


def _alpha_ok(alpha, o_alpha, src_h, w_h, rstd) -> bool:
    """alpha within the absolute 1e-5 of the oracle's; or else within 1e-5 of
    the exact softmax of the logits formed with the kernel's own rstd (held to
    1e-5 relative on its own).  A logit is rstd (w . x), so an rstd off by a
    relative d moves it by d |z|: with a sharp softmax over long rows (|z| in
    the tens) a last-place error of the fp32 rstd alone can move a weight by
    more than 1e-5, while the scores and softmax that follow are exact to
    well within it."""
    a = alpha.cpu().double().numpy()
    if float(np.max(np.abs(a - o_alpha), initial=0.0)) <= TOL_ALPHA_ABS:
        return True
    wx = np.stack([oracle.bf16_to_f64(s) @ w_h.astype(np.float64) for s in src_h], axis=1)  # [T][N]
    z = rstd.cpu().double().numpy() * wx
    e = np.exp(z - z.max(1, keepdims=True))
    a2 = e / e.sum(1, keepdims=True)
    err, err2 = float(np.max(np.abs(a - o_alpha))), float(np.max(np.abs(a - a2)))
    print(f"[fuzz]   alpha: max err {err:.3e} against the oracle, {err2:.3e} at the kernel's own rstd", flush=True)
    return err2 <= TOL_ALPHA_ABS


def _dw_ok(dw, o_dw, src_h, dout_h, w_h, o_rstd, rstd, o_alpha, alpha) -> bool:
    """dw within the operator's relative 1e-2 of the oracle's (near zero where
    the oracle's is zero); or, where the
    derived bound (parity.dw_bound) is itself at least 1e-2 of the oracle's dw
    -- every term of dw rests on weights that the saved fp32 alpha rounds or
    flushes to zero (a token one-hot beyond fp32's range) -- every element
    within that bound."""
    g = dw.cpu().double().numpy()
    if np.linalg.norm(o_dw) == 0:
        return float(np.max(np.abs(g), initial=0.0)) <= 1e-6
    if rel_l2(g, o_dw) <= TOL_DW_REL_L2:
        return True
    b = dw_bound(_t(src_h, DEV), _t(dout_h, DEV), _t(w_h, DEV), _t(o_rstd, DEV), rstd.double(), _t(o_alpha, DEV),
                 alpha.double()).cpu().numpy()
    print(f"[fuzz]   dw: rel-L2 {rel_l2(g, o_dw):.3e}; |bound| / |dw| {np.linalg.norm(b) / np.linalg.norm(o_dw):.3e}, "
          f"max err/bound {float(np.max(np.abs(g - o_dw) / np.maximum(b, 1e-300))):.3e}", flush=True)
    return bool(np.linalg.norm(b) >= TOL_DW_REL_L2 * np.linalg.norm(o_dw) and np.all(np.abs(g - o_dw) <= b))


def _zeros_like_layout(views, dtype=None):
    """Zero gradients in the layout of the source views (same row pitch), in
    the sources' dtype or the given one."""
    out = []
    for v in views:
        dt = v.dtype if dtype is None else dtype
        if v.is_contiguous():
            out.append(torch.zeros(v.shape, dtype=dt, device=v.device))
        else:
            T, D = v.shape
            base = torch.zeros((T, v.stride(0)), dtype=dt, device=v.device)
            out.append(base[:, :D])
    return out


@pytest.mark.parametrize("seed", list(range(96)) + [651, 737, 753, 755, 994, 1902, 3052, 3699, 4057, 5206])  # + wider sweeps' finds
def test_random_configuration(seed):
    rng = np.random.default_rng(1000 + seed)
    N = int(rng.integers(1, 10))
    T = int(rng.integers(1, 200))
    D = 8 * int(rng.choice([1, 2, 7, 64, 125, 513, 896, 1024, 1025, 1536, 2048]))
    eps = float(rng.choice([0.0, 1e-6, 1e-3]))
    kind = "tiny" if N <= 3 and rng.random() < 0.5 else "depth"
    scales = tuple(float(x) for x in np.exp(rng.uniform(-3, 3, 3)))
    w_std = float(rng.choice([0.0, 0.5])) or None  # None: 1/sqrt(D); 0.5: the peaked workload's
    wl = synth.Workload(f"fuzz{seed}", T=T, N=N, D=D, eps=eps, seed=seed, kind=kind, w_std=w_std, tiny_scales=scales)
    layout = str(rng.choice(["stacked", "separate", "interleaved", "padded"]))
    mode = str(rng.choice(["plain", "accumulate", "decode", "update", "f32", "f32acc"]))
    src_h, w_h, dout_h = wl.sources(), wl.w(), wl.dout()
    print(f"[fuzz] seed={seed} N={N} T={T} D={D} eps={eps} kind={kind} layout={layout} mode={mode}", flush=True)
    src = to_dev_bf16(src_h)
    w = torch.from_numpy(w_h).to(DEV)
    dout = to_dev_bf16(dout_h)

    if mode == "update":
        y_h = synth.Workload(f"fuzzy{seed}", T=T, N=1, D=D, seed=seed + 77, kind="tiny",
                             tiny_scales=(0.3,)).sources()[0]
        views = _place(src, "separate" if layout == "stacked" else layout, rng)
        out, rstd, alpha, p_new = ar.attnres_fwd_update(views[:-1], views[-1], to_dev_bf16(y_h), w, eps)
        torch.cuda.synchronize()
        o_out, o_rstd, o_alpha, o_p = oracle.fwd_update(src_h[:-1], src_h[-1], y_h, w_h, eps)
        got_p = p_new.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got_p, o_p)
    elif layout == "stacked" and mode != "decode":
        out, rstd, alpha = ar.attnres_fwd(src, w, eps)
        o_out, o_rstd, o_alpha = oracle.fwd(src_h, w_h, eps)
    else:
        views = _place(src, "separate" if layout == "stacked" else layout, rng)
        if mode == "decode":
            out, rstd, alpha = ar.attnres_fwd_decode(views, w, eps, save_state=True)
        else:
            out, rstd, alpha = ar.attnres_fwd_sources(views, w, eps)
        o_out, o_rstd, o_alpha = oracle.fwd(src_h, w_h, eps)
    torch.cuda.synchronize()
    assert rel_l2(bf16_dev_to_f64(out), o_out) <= TOL_OUT_REL_L2
    assert float(np.max(np.abs(rstd.cpu().double().numpy() / o_rstd - 1))) <= TOL_RSTD_REL
    # the update forward's last source is the updated partial sum
    src_a = src_h if mode != "update" else np.concatenate([src_h[:-1], o_p[None]])
    assert _alpha_ok(alpha, o_alpha, src_a, w_h, rstd)

    if mode in ("f32", "f32acc"):
        # fp32 source gradients, written or accumulated onto seeded fp32 priors
        o_dsrc, o_dw = oracle.bwd(src_h, w_h, eps, dout_h)
        views = _place(src, "separate" if layout == "stacked" else layout, rng)
        grads = _zeros_like_layout(views, torch.float32)
        prior = None
        if mode == "f32acc":
            gen = torch.Generator(device=DEV).manual_seed(seed + 55)
            prior = [torch.randn((T, D), device=DEV, generator=gen) * 0.1 for _ in range(N)]
            for i in range(N):
                grads[i].copy_(prior[i])
        grads, dw = ar.attnres_bwd_sources(dout, views, w, rstd, alpha, dsrcs=grads, accumulate=(mode == "f32acc"))
        torch.cuda.synchronize()
        got = np.stack([g.double().cpu().numpy() for g in grads])
        expect = o_dsrc if prior is None else np.stack([p.double().cpu().numpy() for p in prior]) + o_dsrc
        # fp32 gradients: no bf16 rounding, so each element within the bound of
        # the kernel's fp32 arithmetic (the accumulating mode adds one rounding
        # of the sum); the whole tensor far inside the operator's 1e-2
        xs, gs = _t(src_h, DEV), _t(dout_h, DEV)
        bd = dsrc_bound(xs, gs, _t(w_h, DEV), _t(o_rstd, DEV), rstd.double(), _t(o_alpha, DEV),
                        alpha.double(), _t(o_dsrc, DEV), _t(got, DEV) - (0 if prior is None else _t(expect - o_dsrc, DEV)),
                        out_bits=32)
        if prior is not None:
            bd = bd + U32 * _t(np.abs(expect), DEV)
        ratio = float(((_t(got, DEV) - _t(expect, DEV)).abs() / bd).max())
        print(f"[fuzz]   fp32 gradients: max err/bound {ratio:.3e}, rel-L2 {rel_l2(got, expect):.3e}", flush=True)
        assert ratio <= 1.0, ratio
        assert rel_l2(got, expect) <= 1e-4
        assert _dw_ok(dw, o_dw, src_h, dout_h, w_h, o_rstd, rstd, o_alpha, alpha)
    if mode in ("plain", "accumulate"):
        o_dsrc, o_dw = oracle.bwd(src_h, w_h, eps, dout_h)
        if layout == "stacked":
            dsrc, dw = ar.attnres_bwd(dout, src, w, rstd, alpha)
            got = bf16_dev_to_f64(dsrc)
            expect = o_dsrc
        else:
            views = _place(src, layout, rng)
            grads = _zeros_like_layout(views)
            prior_h = None
            if mode == "accumulate":
                prior_h = synth.Workload(f"fuzzp{seed}", T=T, N=N, D=D, seed=seed + 99, kind="tiny",
                                         tiny_scales=tuple([0.05] * 9)).sources()
                for i in range(N):
                    grads[i].copy_(to_dev_bf16(prior_h[i]))
            grads, dw = ar.attnres_bwd_sources(dout, views, w, rstd, alpha, dsrcs=grads,
                                               accumulate=(mode == "accumulate"))
            got = np.stack([bf16_dev_to_f64(g) for g in grads])
            expect = o_dsrc if prior_h is None else oracle.bf16_to_f64(prior_h) + o_dsrc
        torch.cuda.synchronize()
        assert rel_l2(got, expect) <= TOL_DSRC_REL_L2
        assert _dw_ok(dw, o_dw, src_h, dout_h, w_h, o_rstd, rstd, o_alpha, alpha)


@pytest.mark.parametrize("seed", range(32))
def test_random_block_route(seed):
    """The block-level route on seeded random configurations: block scores of
    n shared sources for L pseudo-queries, block sums (either U layout), and
    the merged forward of a few sub-layers with the partial sum as the last
    source (in half the cases with the fused update of the partial sum,
    checked bit for bit; in half U in the 24-bit format), against the
    oracle's plain forward on all n + 1 sources."""
    rng = np.random.default_rng(5000 + seed)
    n = int(rng.integers(1, 9))
    N = n + 1
    T = int(rng.integers(1, 200))
    D = 8 * int(rng.choice([1, 2, 7, 64, 125, 513, 896, 1024, 1025, 1536, 2048]))
    L = int(rng.integers(1, 41))
    eps = float(rng.choice([0.0, 1e-6, 1e-3]))
    w_std = float(rng.choice([1.0 / np.sqrt(D), 0.5]))
    layout = str(rng.choice(["separate", "interleaved", "padded"]))
    token_major = bool(rng.integers(0, 2))
    wl = synth.Workload(f"fuzzb{seed}", T=T, N=N, D=D, eps=eps, seed=seed, kind="depth")
    src_h = wl.sources()
    W_h = np.stack([synth.normal_f32(D, seed, 300 + l, w_std) for l in range(L)])
    update = bool(rng.integers(0, 2))  # the fused partial-sum update, out of place
    u_format = str(rng.choice(["f32", "f24"]))
    print(f"[fuzz block] seed={seed} n={n} T={T} D={D} L={L} eps={eps} w_std={w_std:.3g} layout={layout} "
          f"token_major={token_major} update={update} U {u_format}", flush=True)
    views = _place(to_dev_bf16(src_h), layout, rng)
    W = torch.from_numpy(W_h).to(DEV)
    rb, zb = ar.attnres_block_scores(views[:n], W, eps)
    U = ar.attnres_block_sums(views[:n], zb, token_major=token_major, u_format=u_format)
    for l in sorted({0, L - 1, int(rng.integers(0, L))}):
        U_l = U[:, l] if token_major else U[l]
        if update:
            y_h = synth.Workload(f"fuzzby{seed}_{l}", T=T, N=1, D=D, seed=seed + l, kind="tiny",
                                 tiny_scales=(0.3,)).sources()[0]
            p_out = _zeros_like_layout([views[n]])[0]
            out, rstd, alpha, p_out = ar.attnres_fwd_merged(U_l, views[n], zb[l], rb, W[l], eps,
                                                            delta=to_dev_bf16(y_h), partial_out=p_out)
            torch.cuda.synchronize()
            o_p = oracle.add_bf16(src_h[n], y_h)
            assert np.array_equal(p_out.contiguous().cpu().view(torch.int16).numpy().view(np.uint16), o_p)
            o_out, o_rstd, o_alpha = oracle.fwd(np.concatenate([src_h[:n], o_p[None]]), W_h[l], eps)
        else:
            out, rstd, alpha = ar.attnres_fwd_merged(U_l, views[n], zb[l], rb, W[l], eps)
            torch.cuda.synchronize()
            o_out, o_rstd, o_alpha = oracle.fwd(src_h, W_h[l], eps)
        assert rel_l2(bf16_dev_to_f64(out), o_out) <= TOL_OUT_REL_L2
        assert float(np.max(np.abs(alpha.cpu().double().numpy() - o_alpha))) <= TOL_ALPHA_ABS
        assert float(np.max(np.abs(rstd.cpu().double().numpy() / o_rstd - 1))) <= TOL_RSTD_REL

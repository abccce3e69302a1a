"""Per-source pointers and gradient accumulation (attnres_fwd_sources /
attnres_bwd_sources): bitwise agreement with the stacked calls, and parity of
the accumulated gradients with the fp64 oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_residuals_depth_amd as ar
import oracle
import synth
from parity import (DEV, TOL_DSRC_REL_L2, TOL_DW_REL_L2, bf16_dev_to_f64, rel_l2, run_gpu, to_dev_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ar.library()


def _bits(t):
    return t.contiguous().view(torch.int16) if t.dtype == torch.bfloat16 else t.contiguous().view(torch.int32)


def _separate(src_stacked):
    """Copy each source into its own allocation (different addresses and order)."""
    return [src_stacked[i].clone() for i in range(src_stacked.shape[0])]


@pytest.mark.parametrize("N,T,D", [(9, 700, 7168), (3, 130, 1000), (5, 40, 12288), (1, 17, 7168)],
                         ids=lambda v: str(v))
def test_sources_match_stacked_bitwise(N, T, D):
    wl = synth.Workload(f"src_N{N}_T{T}_D{D}", T=T, N=N, D=D)
    src = to_dev_bf16(wl.sources())
    w = torch.from_numpy(wl.w()).to(DEV)
    dout = to_dev_bf16(wl.dout())
    out, rstd, alpha, dsrc, dw = run_gpu(src, w, wl.eps, dout)
    srcs = _separate(src)
    o2, r2, a2 = ar.attnres_fwd_sources(srcs, w, wl.eps)
    d2, dw2 = ar.attnres_bwd_sources(dout, srcs, w, r2, a2)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(o2))
    assert torch.equal(_bits(rstd), _bits(r2))
    assert torch.equal(_bits(alpha), _bits(a2))
    for i in range(N):
        assert torch.equal(_bits(dsrc[i]), _bits(d2[i])), i
    assert torch.equal(_bits(dw), _bits(dw2))


def test_repeated_source_pointer():
    """The same tensor may be passed as two sources (reads only)."""
    wl = synth.workload(1, T=64, N=3)
    src = to_dev_bf16(wl.sources())
    w = torch.from_numpy(wl.w()).to(DEV)
    srcs = [src[0], src[1], src[0]]
    stacked = torch.stack(srcs).contiguous()
    o1, r1, a1 = ar.attnres_fwd(stacked, w, wl.eps)
    o2, r2, a2 = ar.attnres_fwd_sources(srcs, w, wl.eps)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o1), _bits(o2)) and torch.equal(_bits(a1), _bits(a2))


# D > 8192 (two vectors per thread) accumulates through a window of old-gradient
# registers: (2, 45, 8200) has no more items than the window, (9, 70, 16384) has 18
@pytest.mark.parametrize("N,T,D", [(9, 512, 7168), (4, 300, 4104), (6, 33, 12288), (1, 20, 7168), (9, 70, 16384),
                                   (2, 45, 8200)],
                         ids=lambda v: str(v))
def test_accumulate_against_oracle(N, T, D):
    wl = synth.Workload(f"acc_N{N}_T{T}_D{D}", T=T, N=N, D=D)
    src_h, dout_h, w_h = wl.sources(), wl.dout(), wl.w()
    # prior gradients of the sources: seeded bf16 values of the size of a step's gradient
    prior = synth.Workload(f"prior_N{N}_T{T}_D{D}", T=T, N=N, D=D, seed=7, kind="tiny",
                           tiny_scales=tuple([0.1] * 9)).sources()
    src = [to_dev_bf16(src_h[i]) for i in range(N)]
    dsrcs = [to_dev_bf16(prior[i]) for i in range(N)]
    w = torch.from_numpy(w_h).to(DEV)
    dout = to_dev_bf16(dout_h)
    out, rstd, alpha = ar.attnres_fwd_sources(src, w, wl.eps)
    dsrcs, dw = ar.attnres_bwd_sources(dout, src, w, rstd, alpha, dsrcs=dsrcs, accumulate=True)
    g32, _ = ar.attnres_bwd_sources(dout, src, w, rstd, alpha, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    # bitwise: the accumulated bf16 gradient is the fp32 sum of the prior and
    # the fp32 increment, rounded once to nearest even
    for i in range(N):
        assert torch.equal(_bits(dsrcs[i]), _bits((to_dev_bf16(prior[i]).float() + g32[i]).to(torch.bfloat16))), i
    o_dsrc, o_dw = oracle.bwd(src_h, w_h, wl.eps, dout_h)
    expect = oracle.bf16_to_f64(prior) + o_dsrc
    got = np.stack([bf16_dev_to_f64(d) for d in dsrcs])
    e_acc = rel_l2(got, expect)
    e_inc = rel_l2(got - oracle.bf16_to_f64(prior), o_dsrc)
    e_dw = rel_l2(dw.cpu().double().numpy(), o_dw)
    print(f"[parity] accumulate N={N} T={T} D={D}: result rel_l2={e_acc:.3e} increment rel_l2={e_inc:.3e} "
          f"dw rel_l2={e_dw:.3e}", flush=True)
    assert e_acc <= TOL_DSRC_REL_L2
    assert e_inc <= TOL_DSRC_REL_L2
    assert e_dw <= TOL_DW_REL_L2


def test_accumulate_twice_equals_sum_of_two_calls():
    """Two accumulating calls with the same inputs add the same increment twice."""
    wl = synth.workload(1, T=256)
    src = to_dev_bf16(wl.sources())
    w = torch.from_numpy(wl.w()).to(DEV)
    dout = to_dev_bf16(wl.dout())
    srcs = _separate(src)
    out, rstd, alpha = ar.attnres_fwd_sources(srcs, w, wl.eps)
    plain, _ = ar.attnres_bwd_sources(dout, srcs, w, rstd, alpha)
    zero = [torch.zeros_like(s) for s in srcs]
    acc, _ = ar.attnres_bwd_sources(dout, srcs, w, rstd, alpha, dsrcs=zero, accumulate=True)
    torch.cuda.synchronize()
    # 0 + dx rounds exactly like dx
    for a, p in zip(acc, plain):
        assert torch.equal(_bits(a), _bits(p))
    acc2, _ = ar.attnres_bwd_sources(dout, srcs, w, rstd, alpha, dsrcs=acc, accumulate=True)
    torch.cuda.synchronize()
    for a, p in zip(acc2, plain):
        assert torch.allclose(a.float(), 2 * p.float(), rtol=8e-3, atol=1e-6)


def _interleave(src_stacked, pad=0):
    """A [T][N][D + pad] cache holding the sources side by side per token, and the
    per-source views into it (row pitch N*(D + pad))."""
    N, T, D = src_stacked.shape
    cache = torch.zeros((T, N, D + pad), dtype=src_stacked.dtype, device=src_stacked.device)
    cache[:, :, :D] = src_stacked.permute(1, 0, 2)
    return cache, [cache[:, i, :D] for i in range(N)]


@pytest.mark.parametrize("N,T,D,pad", [(9, 300, 7168, 0), (4, 65, 1000, 8), (3, 17, 12288, 0), (9, 1, 7168, 0)],
                         ids=lambda v: str(v))
def test_interleaved_sources_match_stacked_bitwise(N, T, D, pad):
    """Sources kept side by side per token ([T][N][D] cache, pitch N*D) and
    gradients written into a cache of the same layout give the stacked calls'
    results bit for bit: forward, decoding forward, backward, accumulating
    backward."""
    wl = synth.Workload(f"inter_N{N}_T{T}_D{D}", T=T, N=N, D=D)
    src = to_dev_bf16(wl.sources())
    w = torch.from_numpy(wl.w()).to(DEV)
    dout = to_dev_bf16(wl.dout())
    out, rstd, alpha, dsrc, dw = run_gpu(src, w, wl.eps, dout)
    cache, views = _interleave(src, pad)
    o2, r2, a2 = ar.attnres_fwd_sources(views, w, wl.eps)
    o3, _, _ = ar.attnres_fwd_decode(views, w, wl.eps)
    dcache, dviews = _interleave(torch.zeros_like(src), pad)
    _, dw2 = ar.attnres_bwd_sources(dout, views, w, r2, a2, dsrcs=dviews)
    acc_cache, acc_views = _interleave(dsrc, pad)  # accumulate onto a copy of the gradients
    ar.attnres_bwd_sources(dout, views, w, r2, a2, dsrcs=acc_views, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(o2)) and torch.equal(_bits(out), _bits(o3))
    assert torch.equal(_bits(rstd), _bits(r2)) and torch.equal(_bits(alpha), _bits(a2))
    assert torch.equal(_bits(dw), _bits(dw2))
    for i in range(N):
        assert torch.equal(_bits(dsrc[i]), _bits(dviews[i])), i
        want = (dsrc[i].float() + dsrc[i].float()).to(torch.bfloat16)  # bf16(x + x) is exact doubling
        assert torch.equal(_bits(want), _bits(acc_views[i])), i
    if pad:
        assert not bool(dcache[:, :, D:].any()) and not bool(cache[:, :, D:].any())  # padding untouched


def test_interleaved_partial_sum_update_in_place():
    """The partial sum as the last slot of an interleaved cache, updated in place."""
    N, T, D = 6, 200, 7168
    wl = synth.Workload(f"inter_upd_N{N}_T{T}_D{D}", T=T, N=N, D=D)
    src = to_dev_bf16(wl.sources())
    w = torch.from_numpy(wl.w()).to(DEV)
    y = to_dev_bf16(synth.Workload("inter_upd_y", T=T, N=1, D=D, seed=5, kind="tiny",
                                   tiny_scales=(0.5,)).sources()[0])
    out1, r1, a1, p1 = ar.attnres_fwd_update([src[i] for i in range(N - 1)], src[N - 1].clone(), y, w, wl.eps)
    cache, views = _interleave(src)
    out2, r2, a2, p2 = ar.attnres_fwd_update(views[:-1], views[-1], y, w, wl.eps)
    torch.cuda.synchronize()
    assert p2.data_ptr() == views[-1].data_ptr()
    assert torch.equal(_bits(p1), _bits(cache[:, N - 1]))
    assert torch.equal(_bits(out1), _bits(out2))
    assert torch.equal(_bits(r1), _bits(r2)) and torch.equal(_bits(a1), _bits(a2))


@pytest.mark.parametrize("N,T,D", [(9, 300, 7168), (4, 65, 1000), (3, 33, 12288), (1, 9, 7168), (9, 40, 16384),
                                   (2, 21, 8200)],
                         ids=lambda v: str(v))
def test_fp32_gradients(N, T, D):
    """fp32 gradients: written (no bf16 rounding: the oracle's dx to fp32
    precision, and bitwise the bf16 mode's values before rounding) and
    accumulated in fp32 onto seeded prior gradients."""
    wl = synth.Workload(f"f32_N{N}_T{T}_D{D}", T=T, N=N, D=D)
    src_h, w_h, dout_h = wl.sources(), wl.w(), wl.dout()
    srcs = [to_dev_bf16(src_h[i]) for i in range(N)]
    w = torch.from_numpy(w_h).to(DEV)
    dout = to_dev_bf16(dout_h)
    out, rstd, alpha = ar.attnres_fwd_sources(srcs, w, wl.eps)
    g32, dw32 = ar.attnres_bwd_sources(dout, srcs, w, rstd, alpha, grad_dtype=torch.float32)
    g16, dw16 = ar.attnres_bwd_sources(dout, srcs, w, rstd, alpha)
    prior = [torch.randn((T, D), device=DEV, generator=torch.Generator(device=DEV).manual_seed(i)) * 0.1
             for i in range(N)]
    acc = [p.clone() for p in prior]
    acc, _ = ar.attnres_bwd_sources(dout, srcs, w, rstd, alpha, dsrcs=acc, accumulate=True)
    torch.cuda.synchronize()
    o_dsrc, o_dw = oracle.bwd(src_h, w_h, wl.eps, dout_h)
    got = np.stack([g.double().cpu().numpy() for g in g32])
    e32 = rel_l2(got, o_dsrc)
    e_acc = rel_l2(np.stack([a.double().cpu().numpy() for a in acc]),
                   np.stack([p.double().cpu().numpy() for p in prior]) + o_dsrc)
    print(f"[parity] fp32 gradients N={N} T={T} D={D}: written rel_l2={e32:.3e} accumulated rel_l2={e_acc:.3e}",
          flush=True)
    assert e32 <= 1e-5
    assert e_acc <= 1e-5
    for i in range(N):
        assert torch.equal(_bits(g32[i].to(torch.bfloat16)), _bits(g16[i])), i
    assert torch.equal(_bits(dw32), _bits(dw16))
    # fp32 accumulation adds exactly the fp32 increment (one fp32 rounding per element)
    for i in range(N):
        assert torch.equal(_bits(acc[i]), _bits(prior[i] + g32[i])), i


def test_fp32_gradients_interleaved():
    """fp32 gradients in a [T][N][D] fp32 cache (pitch N*D) equal dense ones."""
    N, T, D = 6, 128, 7168
    wl = synth.Workload(f"f32_inter_N{N}", T=T, N=N, D=D)
    src = to_dev_bf16(wl.sources())
    w = torch.from_numpy(wl.w()).to(DEV)
    dout = to_dev_bf16(wl.dout())
    srcs = [src[i] for i in range(N)]
    _, rstd, alpha = ar.attnres_fwd_sources(srcs, w, wl.eps)
    dense, _ = ar.attnres_bwd_sources(dout, srcs, w, rstd, alpha, grad_dtype=torch.float32)
    cache = torch.zeros((T, N, D), dtype=torch.float32, device=DEV)
    views = [cache[:, i] for i in range(N)]
    ar.attnres_bwd_sources(dout, srcs, w, rstd, alpha, dsrcs=views)
    ar.attnres_bwd_sources(dout, srcs, w, rstd, alpha, dsrcs=views, accumulate=True)
    torch.cuda.synchronize()
    for i in range(N):
        assert torch.equal(_bits(views[i]), _bits(dense[i] + dense[i])), i


@pytest.mark.slow
def test_interleaved_cache_at_full_size():
    """A [T][N][D] depth-source cache at T = 131072, N = 9, D = 7168 (16.9 GB;
    row addresses reach past 2^32 bytes through the per-token pitch), with the
    gradients written into a [T][N][D] gradient cache: sampled tokens of out,
    alpha, rstd and the gradients against the oracle, and dw over all tokens;
    then fp32 gradients into a [T][N][D] fp32 cache, written and accumulated."""
    from parity import check_tokens, sample_tokens, within_tolerance

    wl = synth.workload(2, N=9, T=131072)
    T, N, D = wl.T, wl.N, wl.D
    print(f"[parity] interleaved full size T={T} N={N} D={D}: generating", flush=True)
    src = wl.sources()
    dout = wl.dout()
    w = wl.w()
    cache = torch.empty((T, N, D), dtype=torch.bfloat16, device=DEV)
    for i in range(N):
        cache[:, i].copy_(to_dev_bf16(src[i]))
    gcache = torch.empty((T, N, D), dtype=torch.bfloat16, device=DEV)
    w_d = torch.from_numpy(w).to(DEV)
    dout_d = to_dev_bf16(dout)
    views = [cache[:, i] for i in range(N)]
    print("[parity] interleaved full size: running fwd+bwd", flush=True)
    out, rstd, alpha = ar.attnres_fwd_sources(views, w_d, wl.eps)
    _, dw = ar.attnres_bwd_sources(dout_d, views, w_d, rstd, alpha, dsrcs=[gcache[:, i] for i in range(N)])
    torch.cuda.synchronize()

    toks = sample_tokens(T)
    s_src = np.ascontiguousarray(src[:, toks])
    o_out, o_rstd, o_alpha = oracle.fwd(s_src, w, wl.eps)
    o_dsrc, _ = oracle.bwd(s_src, w, wl.eps, np.ascontiguousarray(dout[toks]))
    tk = torch.from_numpy(toks).to(DEV)
    gpu = dict(out=bf16_dev_to_f64(out[tk]), rstd=rstd[tk].cpu().double().numpy(),
               alpha=alpha[tk].cpu().double().numpy(), dsrc=bf16_dev_to_f64(gcache[tk].transpose(0, 1)))
    ref = dict(out=o_out, rstd=o_rstd, alpha=o_alpha, dsrc=o_dsrc)
    e = check_tokens({}, wl.name, gpu, ref, (s_src, np.ascontiguousarray(dout[toks]), w))
    print("[parity] interleaved full size: oracle dw over all tokens", flush=True)
    _, o_dw = oracle.bwd(src, w, wl.eps, dout, want_dsrc=False)
    e["dw_rel_l2"] = rel_l2(dw.cpu().double().numpy(), o_dw)
    print("[parity] interleaved full size: " + ", ".join(f"{k}={v:.3e}" for k, v in e.items()), flush=True)
    assert within_tolerance(e), e
    del gcache, out
    torch.cuda.empty_cache()

    # fp32 gradients in a [T][N][D] fp32 cache (33.8 GB): written, then accumulated onto themselves
    g32 = torch.empty((T, N, D), dtype=torch.float32, device=DEV)
    g32_views = [g32[:, i] for i in range(N)]
    for acc in (False, True):
        ar.attnres_bwd_sources(dout_d, views, w_d, rstd, alpha, dsrcs=g32_views, accumulate=acc)
        torch.cuda.synchronize()
        got = g32[tk].transpose(0, 1).double().cpu().numpy()
        err = rel_l2(got, (2.0 if acc else 1.0) * o_dsrc)
        print(f"[parity] interleaved full size, fp32 gradients {'accumulated' if acc else 'written'}: "
              f"rel-L2 {err:.3e}", flush=True)
        assert err <= 1e-5, err
    del cache, g32, dout_d
    torch.cuda.empty_cache()

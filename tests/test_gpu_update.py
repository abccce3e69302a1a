"""The forward fused with the partial-sum update (attnres_fwd_update): the new
partial sum bit-exact against the oracle's correctly rounded bf16(p + y), the
operator's outputs within tolerance of the oracle, and bitwise equal to the
unfused route (update first, then attnres_fwd_sources)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_residuals_depth_amd as ar
import oracle
import synth
from parity import (DEV, TOL_ALPHA_ABS, TOL_OUT_REL_L2, TOL_RSTD_REL, bf16_dev_to_f64, rel_l2, to_dev_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ar.library()


def _bits(t):
    return t.contiguous().view(torch.int16) if t.dtype == torch.bfloat16 else t.contiguous().view(torch.int32)


def _case(N, T, D):
    """N-1 depth sources, the partial sum (scale of the last depth source) and a
    sub-layer output of comparable size, as bf16 bit patterns."""
    wl = synth.Workload(f"upd_N{N}_T{T}_D{D}", T=T, N=N, D=D)
    allsrc = wl.sources()
    delta = synth.Workload(f"upd_delta_T{T}_D{D}", T=T, N=1, D=D, seed=5, kind="tiny",
                           tiny_scales=(0.5,)).sources()[0]
    return wl, allsrc[:N - 1], allsrc[N - 1], delta


@pytest.mark.parametrize("N,T,D", [(9, 300, 7168), (4, 129, 1000), (2, 40, 12288), (1, 17, 7168), (6, 3, 8),
                                   (9, 1, 16384)], ids=lambda v: str(v))
def test_update_against_oracle(N, T, D):
    wl, src_h, p_h, y_h = _case(N, T, D)
    w_h = wl.w()
    srcs = [to_dev_bf16(src_h[i]) for i in range(N - 1)]
    p = to_dev_bf16(p_h)
    y = to_dev_bf16(y_h)
    w = torch.from_numpy(w_h).to(DEV)
    out, rstd, alpha, p_new = ar.attnres_fwd_update(srcs, p, y, w, wl.eps, in_place=False)
    torch.cuda.synchronize()
    o_out, o_rstd, o_alpha, o_p_new = oracle.fwd_update(src_h, p_h, y_h, w_h, wl.eps)
    got_p = p_new.cpu().view(torch.int16).numpy().view(np.uint16)
    mismatches = int(np.count_nonzero(got_p != o_p_new))
    e_out = rel_l2(bf16_dev_to_f64(out), o_out)
    e_alpha = float(np.max(np.abs(alpha.cpu().double().numpy() - o_alpha)))
    e_rstd = float(np.max(np.abs(rstd.cpu().double().numpy() / o_rstd - 1)))
    print(f"[parity] update N={N} T={T} D={D}: partial-sum bit mismatches={mismatches} out rel_l2={e_out:.3e} "
          f"alpha max abs={e_alpha:.3e} rstd max rel={e_rstd:.3e}", flush=True)
    assert mismatches == 0
    assert e_out <= TOL_OUT_REL_L2
    assert e_alpha <= TOL_ALPHA_ABS
    assert e_rstd <= TOL_RSTD_REL


@pytest.mark.parametrize("N,T,D", [(9, 700, 7168), (3, 64, 4104), (1, 5, 1000)], ids=lambda v: str(v))
def test_fused_equals_unfused_and_in_place(N, T, D):
    wl, src_h, p_h, y_h = _case(N, T, D)
    srcs = [to_dev_bf16(src_h[i]) for i in range(N - 1)]
    p = to_dev_bf16(p_h)
    y = to_dev_bf16(y_h)
    w = torch.from_numpy(wl.w()).to(DEV)
    out1, r1, a1, p_new = ar.attnres_fwd_update(srcs, p, y, w, wl.eps, in_place=False)
    out2, r2, a2 = ar.attnres_fwd_sources(srcs + [p_new], w, wl.eps)
    p_inplace = p.clone()
    out3, r3, a3, p3 = ar.attnres_fwd_update(srcs, p_inplace, y, w, wl.eps)
    out4, r4, a4, _ = ar.attnres_fwd_update(srcs, p.clone(), y, w, wl.eps, save_state=False)
    torch.cuda.synchronize()
    assert p3.data_ptr() == p_inplace.data_ptr()
    assert torch.equal(_bits(p3), _bits(p_new))
    for o, r, a in ((out2, r2, a2), (out3, r3, a3)):
        assert torch.equal(_bits(out1), _bits(o))
        assert torch.equal(_bits(r1), _bits(r))
        assert torch.equal(_bits(a1), _bits(a))
    assert r4 is None and a4 is None and torch.equal(_bits(out1), _bits(out4))
    # the partial sum itself was left alone by the out-of-place call
    assert torch.equal(_bits(p), _bits(to_dev_bf16(p_h)))


def test_backward_through_the_updated_partial_sum():
    """The saved state of the fused call drives attnres_bwd_sources with the new
    partial sum as the last source, matching the oracle's gradients."""
    N, T, D = 5, 96, 7168
    wl, src_h, p_h, y_h = _case(N, T, D)
    srcs = [to_dev_bf16(src_h[i]) for i in range(N - 1)]
    w = torch.from_numpy(wl.w()).to(DEV)
    out, rstd, alpha, p_new = ar.attnres_fwd_update(srcs, to_dev_bf16(p_h), to_dev_bf16(y_h), w, wl.eps)
    dout_h = wl.dout()
    dsrcs, dw = ar.attnres_bwd_sources(to_dev_bf16(dout_h), srcs + [p_new], w, rstd, alpha)
    torch.cuda.synchronize()
    p_new_h = oracle.add_bf16(p_h, y_h)
    o_dsrc, o_dw = oracle.bwd(np.concatenate([src_h, p_new_h[None]]), wl.w(), wl.eps, dout_h)
    got = np.stack([bf16_dev_to_f64(d) for d in dsrcs])
    assert rel_l2(got, o_dsrc) <= 1e-2
    assert rel_l2(dw.cpu().double().numpy(), o_dw) <= 1e-2


def test_in_place_update_invalidates_saved_partial_sum():
    """An autograd node that saved the partial sum must refuse its backward once
    attnres_fwd_update has rewritten that tensor in place (the binding bumps the
    tensor's version counter); a partial sum that requires grad is refused."""
    wl, src_h, p_h, y_h = _case(3, 64, 1024)
    srcs = [to_dev_bf16(src_h[i]) for i in range(2)]
    p = to_dev_bf16(p_h)
    y = to_dev_bf16(y_h)
    w = torch.from_numpy(wl.w()).to(DEV).requires_grad_(True)
    out = ar.attnres(srcs + [p], w, wl.eps)  # saves p for its backward
    v0 = p._version
    ar.attnres_fwd_update(srcs, p, y, w.detach(), wl.eps)  # rewrites p in place
    assert p._version > v0
    with pytest.raises(RuntimeError, match="modified by an inplace operation"):
        out.float().sum().backward()
    leaf = to_dev_bf16(p_h).requires_grad_(True)
    with pytest.raises(RuntimeError, match="requires grad"):
        ar.attnres_fwd_update(srcs, leaf, y, w.detach(), wl.eps)
    # not in place: the saved tensor is untouched and the backward runs
    p2 = to_dev_bf16(p_h)
    out2 = ar.attnres(srcs + [p2], w, wl.eps)
    ar.attnres_fwd_update(srcs, p2, y, w.detach(), wl.eps, in_place=False)
    out2.float().sum().backward()
    torch.cuda.synchronize()
    assert w.grad is not None and bool(torch.isfinite(w.grad).all())

"""The autograd wrapper `attnres`: a training step through torch.autograd
gives bitwise the per-source calls' outputs and gradients (the wrapper only
marshals), which match the fp64 oracle; gradients reach a [T][N][D] cache
through its views, and a source used by two calls receives the sum."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_residuals_depth_amd as ar
import oracle
import synth
from parity import DEV, TOL_DSRC_REL_L2, TOL_DW_REL_L2, TOL_OUT_REL_L2, bf16_dev_to_f64, rel_l2, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ar.library()


def _bits(t):
    return t.contiguous().view(torch.int16) if t.dtype == torch.bfloat16 else t.contiguous().view(torch.int32)


def _inputs(N, T, D):
    wl = synth.Workload(f"autograd_N{N}_T{T}_D{D}", T=T, N=N, D=D)
    src_h, w_h, dout_h = wl.sources(), wl.w(), wl.dout()
    return wl, src_h, w_h, dout_h


@pytest.mark.parametrize("N,T,D", [(4, 65, 1000), (9, 300, 7168), (1, 7, 16)], ids=lambda v: str(v))
def test_autograd_step_equals_the_direct_calls(N, T, D):
    wl, src_h, w_h, dout_h = _inputs(N, T, D)
    src = to_dev_bf16(src_h)
    dout = to_dev_bf16(dout_h)
    leaves = [src[i].clone().requires_grad_(True) for i in range(N)]
    w = torch.from_numpy(w_h).to(DEV).requires_grad_(True)
    out = ar.attnres(leaves, w, wl.eps)
    assert out.dtype == torch.bfloat16 and out.requires_grad
    (out.float() * dout.float()).sum().backward()  # d loss / d out = dout exactly (bf16)

    plain = [src[i].clone() for i in range(N)]
    o2, r2, a2 = ar.attnres_fwd_sources(plain, w.detach(), wl.eps)
    d2, dw2 = ar.attnres_bwd_sources(dout, plain, w.detach(), r2, a2)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out.detach()), _bits(o2))
    for i in range(N):
        assert torch.equal(_bits(leaves[i].grad), _bits(d2[i])), i
    assert torch.equal(_bits(w.grad), _bits(dw2))

    o_out, _, _ = oracle.fwd(src_h, w_h, wl.eps)
    o_dsrc, o_dw = oracle.bwd(src_h, w_h, wl.eps, dout_h)
    assert rel_l2(bf16_dev_to_f64(out.detach()), o_out) <= TOL_OUT_REL_L2
    got = np.stack([bf16_dev_to_f64(leaves[i].grad) for i in range(N)])
    assert rel_l2(got, o_dsrc) <= TOL_DSRC_REL_L2
    if N > 1:
        assert rel_l2(w.grad.double().cpu().numpy(), o_dw) <= TOL_DW_REL_L2
    else:
        assert float(w.grad.abs().max()) == 0.0  # one source: alpha = 1 whatever w is


def test_gradients_reach_an_interleaved_cache():
    """Sources as views of one [T][N][D] cache: the cache's gradient holds each
    source's gradient in its slot, bitwise the per-source backward's."""
    N, T, D = 6, 130, 2048
    wl, src_h, w_h, dout_h = _inputs(N, T, D)
    src = to_dev_bf16(src_h)
    dout = to_dev_bf16(dout_h)
    cache = src.permute(1, 0, 2).contiguous().requires_grad_(True)  # [T][N][D]
    w = torch.from_numpy(w_h).to(DEV).requires_grad_(True)
    out = ar.attnres([cache[:, i] for i in range(N)], w, wl.eps)
    out.backward(dout)
    views = [cache.detach()[:, i] for i in range(N)]
    _, r2, a2 = ar.attnres_fwd_sources(views, w.detach(), wl.eps)
    d2, dw2 = ar.attnres_bwd_sources(dout, views, w.detach(), r2, a2)
    torch.cuda.synchronize()
    for i in range(N):
        assert torch.equal(_bits(cache.grad[:, i]), _bits(d2[i])), i
    assert torch.equal(_bits(w.grad), _bits(dw2))


def test_a_source_shared_by_two_calls_gets_the_sum():
    """A block sum read by two sub-layers (two queries): autograd adds the two
    bf16 gradients, i.e. the fp32 sum of the two calls' gradients rounded once
    to bf16."""
    N, T, D = 3, 70, 1024
    wl, src_h, w_h, dout_h = _inputs(N, T, D)
    src = to_dev_bf16(src_h)
    dout = to_dev_bf16(dout_h)
    gen = torch.Generator(device=DEV).manual_seed(5)
    w2 = (torch.randn(D, device=DEV, generator=gen) / D ** 0.5).requires_grad_(True)
    w1 = torch.from_numpy(w_h).to(DEV).requires_grad_(True)
    shared = src[0].clone().requires_grad_(True)
    rest = [src[i].clone() for i in range(1, N)]
    out1 = ar.attnres([shared] + rest, w1, wl.eps)
    out2 = ar.attnres([shared] + rest, w2, wl.eps)
    ((out1.float() + out2.float()) * dout.float()).sum().backward()
    srcs = [shared.detach()] + rest
    g1, _ = ar.attnres_bwd_sources(dout, srcs, w1.detach(), *ar.attnres_fwd_sources(srcs, w1.detach(), wl.eps)[1:])
    g2, _ = ar.attnres_bwd_sources(dout, srcs, w2.detach(), *ar.attnres_fwd_sources(srcs, w2.detach(), wl.eps)[1:])
    torch.cuda.synchronize()
    expect = (g1[0].float() + g2[0].float()).to(torch.bfloat16)
    assert torch.equal(_bits(shared.grad), _bits(expect))

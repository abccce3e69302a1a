"""The split backward's two routes to another slice's partial sums agree bit
for bit: the ring exchange (default poll bound) and the recomputation from
HBM that a workgroup takes when a word does not arrive (forced here from the
host with a poll bound of 0 -- every word -- or 1 -- a mix of both routes).
Every kernel still exits normally: the bound only shortens a bounded wait."""
from __future__ import annotations

import pytest
import torch

import attention_residuals_depth_amd as ar
import synth
from parity import DEV, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ar.library()


@pytest.fixture
def spin():
    """Sets the poll bound for one test and restores the default afterwards."""
    def set_(polls):
        ar.set_split_spin(polls)
    yield set_
    ar.set_split_spin(ar.SPLIT_SPIN_DEFAULT)


def _bits(t):
    return t.contiguous().view(torch.int16) if t.dtype == torch.bfloat16 else t.contiguous().view(torch.int32)


def _inputs(N, T, D, seed):
    wl = synth.Workload("split_route", T, N, D, seed=seed)
    src = to_dev_bf16(wl.sources())
    w = torch.from_numpy(wl.w()).to(DEV)
    dout = to_dev_bf16(wl.dout())
    out, rstd, alpha = ar.attnres_fwd(src, w, wl.eps)
    return src, w, dout, rstd, alpha


# (N, T, D), all where the split backward runs (ATTNRES_BWD_SPLIT): the full
# width (7 slices), a ragged last slice (D/8 = 513 vectors, the fifth slice has
# one; 895 vectors, the seventh has 127), one slice, and token counts that
# leave the last 4-token span ragged
SHAPES = [(9, 131, 7168), (8, 66, 4104), (1, 5, 8), (9, 4, 1024), (8, 257, 7160), (3, 70, 1024)]


def test_shapes_take_the_split_backward():
    assert all(ar.bwd_split(N, D) for N, _, D in SHAPES)


@pytest.mark.parametrize("N,T,D", SHAPES, ids=lambda v: str(v))
@pytest.mark.parametrize("polls", [0, 1])
def test_recompute_route_is_bitwise_the_exchange(N, T, D, polls, spin):
    src, w, dout, rstd, alpha = _inputs(N, T, D, 0)
    ref_dsrc, ref_dw = ar.attnres_bwd(dout, src, w, rstd, alpha)
    torch.cuda.synchronize()
    spin(polls)
    dsrc, dw = ar.attnres_bwd(dout, src, w, rstd, alpha)
    torch.cuda.synchronize()
    assert torch.equal(_bits(dsrc), _bits(ref_dsrc))
    assert torch.equal(_bits(dw), _bits(ref_dw))


@pytest.mark.parametrize("accumulate,gdt", [(True, torch.bfloat16), (False, torch.float32), (True, torch.float32)],
                         ids=["acc_bf16", "f32", "acc_f32"])
def test_recompute_route_in_every_gradient_mode(accumulate, gdt, spin):
    N, T, D = 9, 70, 7168
    src, w, dout, rstd, alpha = _inputs(N, T, D, 1)
    srcs = [src[i] for i in range(N)]
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    base = [torch.randn((T, D), generator=g, device=DEV).to(gdt) for _ in range(N)]
    a = [b.clone() for b in base]
    ref, ref_dw = ar.attnres_bwd_sources(dout, srcs, w, rstd, alpha, dsrcs=a, accumulate=accumulate)
    torch.cuda.synchronize()
    spin(0)
    b = [x.clone() for x in base]
    got, dw = ar.attnres_bwd_sources(dout, srcs, w, rstd, alpha, dsrcs=b, accumulate=accumulate)
    torch.cuda.synchronize()
    for i in range(N):
        assert torch.equal(_bits(got[i]), _bits(ref[i])), i
    assert torch.equal(_bits(dw), _bits(ref_dw))

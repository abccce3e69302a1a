"""The split backward runs its spans (4 tokens side by side) in chunks of
ATTNRES_SPLIT_CHUNK_SPANS, folding each chunk's dw partial rows before the
next chunk reuses the workspace.  These tests cross chunk boundaries (T just
above one and two chunks, a last chunk of a single span and of a ragged span)
at small D, so the oracle compares every element: dsources element by element
within their derived bounds, dw over the whole batch.  They also check that the
chunked result is deterministic, that a token's gradient rows do not depend on
which chunk it falls in, and that the recompute route of the exchange gives
the same bits across chunks."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_residuals_depth_amd as ar
import synth
from parity import DEV, check_tokens, full_compare, to_dev_bf16, within_tolerance

pytestmark = pytest.mark.gpu

CHUNK_TOKENS = ar.SPLIT_CHUNK_SPANS * ar.SPLIT_TOKENS  # 32768


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ar.library()


# (N, T, D): one span past a chunk, a ragged one-token span past a chunk, two
# whole chunks plus a partial third, a wider row (two slices)
SHAPES = [(3, CHUNK_TOKENS + 4, 64), (2, CHUNK_TOKENS + 1, 8), (4, 2 * CHUNK_TOKENS + 13, 16),
          (9, CHUNK_TOKENS + 7, 1032)]


@pytest.mark.parametrize("N,T,D", SHAPES, ids=lambda v: str(v))
def test_chunked_backward_matches_the_oracle(N, T, D):
    wl = synth.Workload(f"chunks_N{N}_T{T}_D{D}", T=T, N=N, D=D)
    print(f"[chunks] N={N} T={T} D={D}", flush=True)
    gpu, ref, inputs = full_compare(wl)
    e = check_tokens({}, wl.name, gpu, ref, inputs)
    print("[chunks] " + ", ".join(f"{k}={v:.3e}" for k, v in e.items()), flush=True)
    assert within_tolerance(e), e


def _inputs(N, T, D, seed=0):
    wl = synth.Workload("chunks", T=T, N=N, D=D, seed=seed)
    src = to_dev_bf16(wl.sources())
    w = torch.from_numpy(wl.w()).to(DEV)
    dout = to_dev_bf16(wl.dout())
    _, rstd, alpha = ar.attnres_fwd(src, w, wl.eps)
    return src, w, dout, rstd, alpha


def test_chunked_backward_is_deterministic_and_rows_do_not_depend_on_the_chunk():
    N, T, D = 3, 2 * CHUNK_TOKENS + 9, 64
    src, w, dout, rstd, alpha = _inputs(N, T, D)
    d1, w1 = ar.attnres_bwd(dout, src, w, rstd, alpha)
    d2, w2 = ar.attnres_bwd(dout, src, w, rstd, alpha)
    torch.cuda.synchronize()
    assert torch.equal(d1.view(torch.int16), d2.view(torch.int16))
    assert torch.equal(w1.view(torch.int32), w2.view(torch.int32))
    # tokens of the second and third chunk, run on their own as a small batch
    for t0 in (CHUNK_TOKENS - 3, 2 * CHUNK_TOKENS):
        n = 9
        s = src[:, t0:t0 + n].contiguous()
        ds, _ = ar.attnres_bwd(dout[t0:t0 + n].contiguous(), s, w, rstd[t0:t0 + n].contiguous(),
                               alpha[t0:t0 + n].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(ds.view(torch.int16), d1[:, t0:t0 + n].view(torch.int16)), t0


def test_recompute_route_across_chunks():
    N, T, D = 2, CHUNK_TOKENS + 6, 1024
    src, w, dout, rstd, alpha = _inputs(N, T, D, seed=3)
    ref_d, ref_w = ar.attnres_bwd(dout, src, w, rstd, alpha)
    torch.cuda.synchronize()
    try:
        ar.set_split_spin(0)
        d, dw = ar.attnres_bwd(dout, src, w, rstd, alpha)
        torch.cuda.synchronize()
    finally:
        ar.set_split_spin(ar.SPLIT_SPIN_DEFAULT)
    assert torch.equal(d.view(torch.int16), ref_d.view(torch.int16))
    assert torch.equal(dw.view(torch.int32), ref_w.view(torch.int32))


@pytest.mark.parametrize("accumulate,gdt", [(True, torch.bfloat16), (False, torch.float32), (True, torch.float32)],
                         ids=["acc_bf16", "f32", "acc_f32"])
def test_gradient_modes_across_chunks(accumulate, gdt):
    """The per-source backward's other gradient modes across a chunk boundary, on
    an interleaved [T][N][D] cache: the written or accumulated gradients minus
    their prior contents against the oracle's, element by element within the
    overwriting backward's derived bound (tests/parity.py) plus, when a bf16
    sum is rounded, half an ulp of that sum; dw over the whole batch."""
    import oracle
    from parity import bf16_ulp, dsrc_bound
    N, T, D = 8, CHUNK_TOKENS + 5, 1040
    assert ar.bwd_split(N, D)
    wl = synth.Workload("chunks_modes", T=T, N=N, D=D, seed=7)
    src_h, w_h, dout_h = wl.sources(), wl.w(), wl.dout()
    cache = to_dev_bf16(np.ascontiguousarray(src_h.transpose(1, 0, 2)))  # [T][N][D]
    views = [cache[:, i] for i in range(N)]
    w = torch.from_numpy(w_h).to(DEV)
    dout = to_dev_bf16(dout_h)
    _, rstd, alpha = ar.attnres_fwd_sources(views, w, wl.eps)
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    prior = (torch.randn((T, N, D), generator=g, device=DEV) * 0.01).to(gdt)
    grads = prior.clone()
    _, dw = ar.attnres_bwd_sources(dout, views, w, rstd, alpha, dsrcs=[grads[:, i] for i in range(N)],
                                   accumulate=accumulate)
    torch.cuda.synchronize()
    _, o_rstd, o_alpha = oracle.fwd(src_h, w_h, wl.eps)
    o_dsrc, o_dw = oracle.bwd(src_h, w_h, wl.eps, dout_h)
    res = grads.double().permute(1, 0, 2)                                    # [N][T][D] on the device
    got = res - (prior.double().permute(1, 0, 2) if accumulate else 0.0)
    ref = torch.from_numpy(o_dsrc).to(DEV)
    x = cache.double().permute(1, 0, 2)
    bound = dsrc_bound(x, dout.double(), w.double(), torch.from_numpy(o_rstd).to(DEV), rstd.double(),
                       torch.from_numpy(o_alpha).to(DEV), alpha.double(), ref, got)
    if accumulate and gdt == torch.bfloat16:
        bound = bound + 0.5 * bf16_ulp(res.abs())
    ratio = float(((got - ref).abs() / bound).max())
    print(f"[chunks] {gdt} accumulate={accumulate}: max err / bound {ratio:.3f}", flush=True)
    assert ratio <= 1.0
    dw_rel = float(np.linalg.norm(dw.cpu().double().numpy() - o_dw) / np.linalg.norm(o_dw))
    assert dw_rel <= 1e-5, dw_rel

"""Block-batched scores (attnres_block_scores, MFMA) and the forward from those
scores (attnres_fwd_scored) against the fp64 oracle, through the C ABI.

Every 12 layers form one AttnRes block; the embedding and the completed block
sums are the same sources before every alpha of the block, each sub-layer with
its own pseudo-query (architecture figure of "Kimi K3 模型结构（10）").

Tolerances.  rstd: 1e-5 relative (an fp32 sum of exact bf16 squares; the
kernel sums each lane's channels in runs of 16 k-steps).  z: element by element
|z - z_ref| <= G r sum_d |W_ld x_d| + |z_ref| (|r - r_ref| / r_ref + 2u), with
G = 256 u (u = 2^-24): the dot is an fp32 accumulation of exact bf16 products
(the queries split exactly into three bf16 parts) in chains of at most
16 k-steps x 3 parts plus the chunk sums; a transposed operand, a wrong row or
a dropped part gives errors of the order of z itself.  The scored forward
meets the operator's own bars (out rel-L2 5e-3 and the element-wise out bound,
alpha 1e-5 absolute, rstd 1e-5 relative) against the plain oracle forward on
all N sources.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_residuals_depth_amd as ar
import oracle
import synth
from parity import DEV, Accum, TOL_ALPHA_ABS, TOL_OUT_REL_L2, TOL_RSTD_REL, to_dev_bf16, within_tolerance

pytestmark = pytest.mark.gpu
U = 2.0 ** -24
GAMMA_BLOCK = 256 * U


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ar.library()


def _queries(D, L, seed, std=None):
    """L pseudo-queries [L][D] fp32 from the seeded generator."""
    std = 1.0 / np.sqrt(D) if std is None else std
    return np.stack([synth.normal_f32(D, seed, 50 + l, std) for l in range(L)])


def _z_ratio(bits, W, eps, r_gpu, z_gpu, r_ref, z_ref):
    """max |z_gpu - z_ref| / bound (see the module docstring); bits [n][T][D]."""
    x = torch.from_numpy(oracle.bf16_to_f64(bits)).to(DEV)                     # [n][T][D]
    absdot = torch.matmul(x.abs(), torch.from_numpy(np.abs(W).astype(np.float64)).to(DEV).T)  # [n][T][L]
    rr = torch.from_numpy(r_ref).to(DEV)                                       # [T][n]
    dr = (torch.from_numpy(r_gpu).to(DEV) - rr).abs() / rr
    zr = torch.from_numpy(z_ref).to(DEV)                                       # [L][T][n]
    bound = GAMMA_BLOCK * rr.T[:, :, None] * absdot                            # [n][T][L]
    bound = bound.permute(2, 1, 0) + zr.abs() * (dr[None] + 2 * U) + 1e-30
    return float(((torch.from_numpy(z_gpu).to(DEV) - zr).abs() / bound).max())


def _block_case(n, T, D, L, eps=1e-6, seed=0, w_std=None, interleave=False):
    wl = synth.Workload(f"blk_n{n}_T{T}_D{D}", T=T, N=n, D=D, seed=seed)
    bits = wl.sources()
    W = _queries(D, L, seed, w_std)
    if interleave:  # the n sources side by side per token, one [T][n][D] cache
        cache = torch.empty((T, n, D), dtype=torch.bfloat16, device=DEV)
        for i in range(n):
            cache[:, i].copy_(to_dev_bf16(bits[i]))
        srcs = [cache[:, i] for i in range(n)]
    else:
        srcs = [to_dev_bf16(bits[i]) for i in range(n)]
    r, z = ar.attnres_block_scores(srcs, torch.from_numpy(W).to(DEV), eps)
    torch.cuda.synchronize()
    return wl, bits, W, srcs, r.cpu().double().numpy(), z.cpu().double().numpy()


@pytest.mark.parametrize("n,T,D,L,inter", [(8, 300, 7168, 24, False), (3, 70, 1000, 5, False), (1, 17, 64, 1, False),
                                           (9, 40, 7176, 33, False), (4, 257, 16384, 16, False),
                                           (8, 130, 7168, 24, True), (2, 1, 7168, 64, False)],
                         ids=lambda v: str(v))
def test_block_scores_against_oracle(n, T, D, L, inter):
    wl, bits, W, _, r, z = _block_case(n, T, D, L, interleave=inter)
    o_r, o_z = oracle.block_scores(bits, W, wl.eps)
    e_r = float(np.max(np.abs(r / o_r - 1)))
    ratio = _z_ratio(bits, W, wl.eps, r, z, o_r, o_z)
    print(f"[block] n={n} T={T} D={D} L={L} interleaved={inter}: rstd max rel {e_r:.3e}, z max err/bound "
          f"{ratio:.3e}, z max abs err {np.max(np.abs(z - o_z)):.3e}", flush=True)
    assert e_r <= TOL_RSTD_REL
    assert ratio <= 1.0


def test_block_scores_are_batch_invariant():
    """A token's rstd and scores do not depend on the batch it is in (rows are
    independent in the product)."""
    _, bits, W, srcs, r, z = _block_case(5, 300, 7168, 24)
    sub = [s[37:101] for s in srcs]
    r2, z2 = ar.attnres_block_scores(sub, torch.from_numpy(W).to(DEV), 1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(r2.cpu().double().numpy(), r[37:101])
    assert np.array_equal(z2.cpu().double().numpy(), z[:, 37:101])


def _scored_vs_plain_oracle(N, T, D, L, w_std=None, subs=(0,), chunk=4096):
    """The block's shared sources are the first N-1; the partial sum is the last.
    Each listed sub-layer's scored forward is compared with the plain oracle
    forward on all N sources (every token, element by element for out)."""
    wl = synth.workload(1, N=N, T=T) if D == synth.D_MODEL else synth.Workload("scored", T=T, N=N, D=D)
    bits = wl.sources()
    W = _queries(D, L, 3, w_std)
    srcs = [to_dev_bf16(bits[i]) for i in range(N)]
    Wd = torch.from_numpy(W).to(DEV)
    rb, zb = ar.attnres_block_scores(srcs[:-1], Wd, wl.eps)
    errs = []
    for l in subs:
        out, rstd, alpha = ar.attnres_fwd_scored(srcs, zb[l], rb, Wd[l], wl.eps)
        torch.cuda.synchronize()
        acc = Accum(DEV)
        for t0 in range(0, T, chunk):
            t1 = min(T, t0 + chunk)
            xs = np.ascontiguousarray(bits[:, t0:t1])
            o_out, o_rstd, o_alpha = oracle.fwd(xs, W[l], wl.eps)
            acc.update(xs, None, W[l], dict(out=out[t0:t1], rstd=rstd[t0:t1], alpha=alpha[t0:t1]),
                       dict(out=o_out, rstd=o_rstd, alpha=o_alpha))
        e = acc.result()
        print(f"[scored] N={N} T={T} D={D} sub-layer {l}: " + ", ".join(f"{k}={v:.3e}" for k, v in e.items()),
              flush=True)
        errs.append(e)
    return errs


@pytest.mark.parametrize("N,T,D", [(9, 300, 7168), (2, 65, 1000), (5, 129, 12288)], ids=lambda v: str(v))
def test_scored_forward_against_oracle(N, T, D):
    for e in _scored_vs_plain_oracle(N, T, D, L=24, subs=(0, 7, 23)):
        assert within_tolerance(e), e


def test_scored_forward_peaked_softmax():
    """Pseudo-queries ~ N(0, 0.5): scores of std ~40, nearly one-hot weights."""
    for e in _scored_vs_plain_oracle(9, 4096, 7168, L=24, w_std=0.5, subs=(0, 23)):
        assert within_tolerance(e), e
        assert e["alpha_max_abs"] <= TOL_ALPHA_ABS


def test_scored_forward_feeds_the_backward():
    """The scored forward's rstd/alpha drive attnres_bwd_sources like the plain
    forward's: gradients within the bars of the oracle's."""
    N, T, D = 9, 200, 7168
    wl = synth.workload(1, N=N, T=T)
    bits, dout = wl.sources(), wl.dout()
    W = _queries(D, 4, 3)
    srcs = [to_dev_bf16(bits[i]) for i in range(N)]
    Wd = torch.from_numpy(W).to(DEV)
    rb, zb = ar.attnres_block_scores(srcs[:-1], Wd, wl.eps)
    out, rstd, alpha = ar.attnres_fwd_scored(srcs, zb[2], rb, Wd[2], wl.eps)
    dsrcs, dw = ar.attnres_bwd_sources(to_dev_bf16(dout), srcs, Wd[2], rstd, alpha)
    torch.cuda.synchronize()
    o_dsrc, o_dw = oracle.bwd(bits, W[2], wl.eps, dout)
    got = np.stack([d.float().cpu().double().numpy() for d in dsrcs])
    rel = np.linalg.norm(got - o_dsrc) / np.linalg.norm(o_dsrc)
    rel_dw = np.linalg.norm(dw.cpu().double().numpy() - o_dw) / np.linalg.norm(o_dw)
    assert rel <= 1e-2 and rel_dw <= 1e-2, (rel, rel_dw)


@pytest.mark.slow
def test_block_full_size_T32768():
    """The N-sweep size with the model's last block: 8 shared sources, 24
    sub-layers; z of four sub-layers on every token against the oracle, then
    two sub-layers' scored forwards on every token."""
    n, T, D, L = 8, 32768, 7168, 24
    print(f"[block] full size n={n} T={T} L={L}: generating", flush=True)
    wl, bits, W, srcs, r, z = _block_case(n, T, D, L)
    print("[block] full size: oracle block scores for four sub-layers", flush=True)
    o_r, o_z = oracle.block_scores(bits, W[[0, 5, 17, 23]], wl.eps)
    e_r = float(np.max(np.abs(r / o_r - 1)))
    ratio = _z_ratio(bits, W[[0, 5, 17, 23]], wl.eps, r, z[[0, 5, 17, 23]], o_r, o_z)
    print(f"[block] full size: rstd max rel {e_r:.3e}, z max err/bound {ratio:.3e}", flush=True)
    assert e_r <= TOL_RSTD_REL and ratio <= 1.0
    del srcs
    torch.cuda.empty_cache()
    for e in _scored_vs_plain_oracle(9, T, D, L=24, subs=(0, 23)):
        assert within_tolerance(e), e

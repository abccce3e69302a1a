"""Block-batched shared sums (attnres_block_sums) and the forward from them
(attnres_fwd_merged) against the fp64 oracle, through the C ABI.

Within a block only the last source, the current partial sum, changes from one
sub-layer to the next (architecture figure of "Kimi K3 模型结构（10）"), and the
weighted sum is linear in the sources: the shared sources' part of every
sub-layer's weighted sum is formed once per block, and each sub-layer's
forward then reads its shared sum and the partial sum alone.

Tolerances.  U: element by element within ``parity.sums_bound`` (the fp32
weights' exponentials and the n-term fp32 sum, doubled), both sides given the
same fp32 scores.  The merged forward meets the operator's own bars against
the plain oracle forward on all N sources (out rel-L2 5e-3, alpha 1e-5
absolute, rstd 1e-5 relative) and, element by element, ``merged_out_bound``:
the plain forward's bound plus the difference between a shared source's
weight through the rescaled sum and the saved alpha.

The 24-bit element format of U (each fp32 sum rounded to nearest even on a
16-bit significand, three bytes kept): its bytes are checked bit for bit
against the oracle's encoding (oracle.round24, pinned by hand-worked cases and
exact rational rounding) of the library's fp32 sums; the merged forward on it
bit for bit against the merged forward on the decoded values given as fp32;
and the chain against the oracle within merged_out_bound plus the format's
2^-16 relative error on the shared part.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_residuals_depth_amd as ar
import oracle
import synth
from parity import DEV, U24, Accum, TOL_ALPHA_ABS, _t, sums_bound, to_dev_bf16, within_tolerance

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ar.library()


def _queries(D, L, seed, std=None):
    """L pseudo-queries [L][D] fp32 from the seeded generator."""
    std = 1.0 / np.sqrt(D) if std is None else std
    return np.stack([synth.normal_f32(D, seed, 60 + l, std) for l in range(L)])


def _sources(n, T, D, seed=0):
    wl = synth.Workload(f"sums_n{n}_T{T}_D{D}", T=T, N=n, D=D, seed=seed)
    return wl, wl.sources()


def _u_rows(U, token_major):
    """U as [L][T][D] (a view)."""
    return U.transpose(0, 1) if token_major else U


@pytest.mark.parametrize("n,T,D,L,tmaj,w_std", [(8, 300, 7168, 24, False, None), (8, 130, 7168, 24, True, None),
                                                 (3, 70, 1000, 5, False, None), (1, 17, 64, 1, False, None),
                                                 (9, 40, 7176, 33, True, None), (4, 257, 16384, 16, False, None),
                                                 (2, 1, 7168, 64, False, None), (5, 33, 512, 7, True, None),
                                                 (8, 200, 7168, 24, False, 0.5)],
                         ids=lambda v: str(v))
def test_block_sums_against_oracle(n, T, D, L, tmaj, w_std):
    """Every element of U against the oracle's sums of the same fp32 scores
    (the oracle's own block scores, rounded to fp32, given to both sides)."""
    wl, bits = _sources(n, T, D)
    W = _queries(D, L, 1, w_std)
    _, zo = oracle.block_scores(bits, W, wl.eps)
    z32 = zo.astype(np.float32)
    srcs = [to_dev_bf16(bits[i]) for i in range(n)]
    print(f"[sums] n={n} T={T} D={D} L={L} token_major={tmaj} w_std={w_std}", flush=True)
    U = ar.attnres_block_sums(srcs, torch.from_numpy(z32).to(DEV), token_major=tmaj)
    torch.cuda.synchronize()
    Uo = oracle.block_sums(bits, z32.astype(np.float64))
    Ug = _u_rows(U, tmaj).double()
    Ur = torch.from_numpy(Uo).to(DEV)
    x = _t(bits, DEV)
    bound = sums_bound(x, torch.from_numpy(z32.astype(np.float64)).to(DEV))
    ratio = float(((Ug - Ur).abs() / (bound + 1e-300)).max())
    rel = float((Ug - Ur).norm() / Ur.norm())
    print(f"[sums]   max err/bound {ratio:.3e}, rel-L2 {rel:.3e}", flush=True)
    assert ratio <= 1.0


def test_block_sums_layouts_and_batch_agree_bitwise():
    """Token-major and sub-layer-major U hold the same bits; a token's rows do
    not depend on the batch it is in; interleaved [T][n][D] sources give the
    same bits as separate ones."""
    n, T, D, L = 6, 200, 7168, 24
    wl, bits = _sources(n, T, D, seed=3)
    W = _queries(D, L, 2)
    srcs = [to_dev_bf16(bits[i]) for i in range(n)]
    _, z = ar.attnres_block_scores(srcs, torch.from_numpy(W).to(DEV), wl.eps)
    U1 = ar.attnres_block_sums(srcs, z)
    U2 = ar.attnres_block_sums(srcs, z, token_major=True)
    cache = torch.empty((T, n, D), dtype=torch.bfloat16, device=DEV)
    for i in range(n):
        cache[:, i].copy_(srcs[i])
    U3 = ar.attnres_block_sums([cache[:, i] for i in range(n)], z)
    U4 = ar.attnres_block_sums([s[37:101] for s in srcs], z[:, 37:101].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(U1, U2.transpose(0, 1))
    assert torch.equal(U1, U3)
    assert torch.equal(U1[:, 37:101], U4)


def _chain(N, T, D, L, w_std=None, subs=(0,), seed=0, chunk=2048, u_format="f32"):
    """GPU: block scores -> block sums -> each listed sub-layer's merged forward,
    all on the device; compared with the plain oracle forward on all N
    sources (the shared ones first, the partial sum last), every token."""
    wl = synth.workload(1, N=N, T=T) if D == synth.D_MODEL else synth.Workload("merged", T=T, N=N, D=D, seed=seed)
    bits = wl.sources()
    W = _queries(D, L, 3 + seed, w_std)
    srcs = [to_dev_bf16(bits[i]) for i in range(N)]
    Wd = torch.from_numpy(W).to(DEV)
    rb, zb = ar.attnres_block_scores(srcs[:-1], Wd, wl.eps)
    U = ar.attnres_block_sums(srcs[:-1], zb, u_format=u_format)
    errs = []
    for l in subs:
        print(f"[merged] N={N} T={T} D={D} sub-layer {l} w_std={w_std} U {u_format}", flush=True)
        out, rstd, alpha = ar.attnres_fwd_merged(U[l], srcs[-1], zb[l], rb, Wd[l], wl.eps)
        torch.cuda.synchronize()
        acc = Accum(DEV)
        for t0 in range(0, T, chunk):
            t1 = min(T, t0 + chunk)
            xs = np.ascontiguousarray(bits[:, t0:t1])
            o_out, o_rstd, o_alpha = oracle.fwd(xs, W[l], wl.eps)
            acc.update(xs, None, W[l], dict(out=out[t0:t1], rstd=rstd[t0:t1], alpha=alpha[t0:t1]),
                       dict(out=o_out, rstd=o_rstd, alpha=o_alpha, merged=True,
                            u_rel=U24 if u_format == "f24" else 0.0))
        e = acc.result()
        print(f"[merged]   " + ", ".join(f"{k}={v:.3e}" for k, v in e.items()), flush=True)
        errs.append(e)
    return errs


@pytest.mark.parametrize("N,T,D", [(9, 300, 7168), (2, 65, 1000), (5, 129, 12288), (9, 77, 512), (4, 1, 7168)],
                         ids=lambda v: str(v))
def test_merged_forward_against_oracle(N, T, D):
    for e in _chain(N, T, D, L=24, subs=(0, 7, 23)):
        assert within_tolerance(e), e


@pytest.mark.parametrize("N,T,D", [(9, 300, 7168), (2, 65, 1000), (5, 129, 12288), (9, 77, 512), (3, 45, 7176)],
                         ids=lambda v: str(v))
def test_merged_forward_f24_against_oracle(N, T, D):
    for e in _chain(N, T, D, L=24, subs=(0, 7, 23), u_format="f24"):
        assert within_tolerance(e), e


@pytest.mark.parametrize("n,T,D,L,tmaj", [(8, 300, 7168, 24, False), (8, 130, 7168, 24, True), (9, 40, 7176, 33, True),
                                          (4, 257, 16384, 16, False), (1, 17, 64, 1, False), (3, 70, 1000, 5, True)],
                         ids=lambda v: str(v))
def test_block_sums_f24_is_the_rounded_fp32(n, T, D, L, tmaj):
    """U in the 24-bit format holds exactly the oracle's encoding (oracle.round24)
    of the library's own fp32 sums, every byte, in both layouts; decode_u24
    reads them as the oracle's decode24 does; and the decoded sums lie within
    the fp32 bound plus the format's rounding of the oracle's sums."""
    wl, bits = _sources(n, T, D, seed=4)
    W = _queries(D, L, 7)
    srcs = [to_dev_bf16(bits[i]) for i in range(n)]
    print(f"[sums f24] n={n} T={T} D={D} L={L} token_major={tmaj}", flush=True)
    _, z = ar.attnres_block_scores(srcs, torch.from_numpy(W).to(DEV), wl.eps)
    U32 = ar.attnres_block_sums(srcs, z, token_major=tmaj)
    Ub = ar.attnres_block_sums(srcs, z, token_major=tmaj, u_format="f24")
    torch.cuda.synchronize()
    assert Ub.dtype == torch.uint8 and Ub.shape == U32.shape + (3,)
    want = oracle.round24(U32.cpu().numpy())
    got = Ub.cpu().numpy()
    assert np.array_equal(got, want), f"{int((got != want).any(-1).sum())} elements differ"
    dec = ar.decode_u24(Ub)
    assert np.array_equal(dec.cpu().numpy().view(np.uint32), oracle.decode24(want).view(np.uint32))
    Uo = oracle.block_sums(bits, z.cpu().double().numpy())
    Ur = torch.from_numpy(Uo).to(DEV)
    Ug = _u_rows(dec, tmaj).double()
    bound = sums_bound(_t(bits, DEV), z.double()) + U24 * Ug.abs()
    ratio = float(((Ug - Ur).abs() / (bound + 1e-300)).max())
    print(f"[sums f24]   max err/bound {ratio:.3e}", flush=True)
    assert ratio <= 1.0


@pytest.mark.parametrize("update", [False, True], ids=["plain", "update"])
def test_merged_f24_is_the_merged_forward_on_the_decoded_sums(update):
    """The merged forward reading 24-bit U gives bitwise the outputs of the
    merged forward reading the decoded values as fp32 (both layouts; with the
    fused update too): the format changes only what is stored."""
    N, T, D, L = 9, 257, 7168, 24
    wl = synth.workload(1, N=N, T=T)
    bits = wl.sources()
    W = torch.from_numpy(_queries(D, L, 8)).to(DEV)
    srcs = [to_dev_bf16(bits[i]) for i in range(N)]
    rb, zb = ar.attnres_block_scores(srcs[:-1], W, wl.eps)
    Ub = ar.attnres_block_sums(srcs[:-1], zb, u_format="f24")
    Ubt = ar.attnres_block_sums(srcs[:-1], zb, token_major=True, u_format="f24")
    dec = ar.decode_u24(Ub).contiguous()
    y = to_dev_bf16(synth.Workload("merged_y24", T=T, N=1, D=D, seed=11, kind="tiny",
                                   tiny_scales=(0.3,)).sources()[0]) if update else None
    for l in (0, 12, 23):
        kw = {} if not update else dict(delta=y, in_place=False)
        r24 = ar.attnres_fwd_merged(Ub[l], srcs[-1], zb[l], rb, W[l], wl.eps, **kw)
        r24t = ar.attnres_fwd_merged(Ubt[:, l], srcs[-1], zb[l], rb, W[l], wl.eps, **kw)
        r32 = ar.attnres_fwd_merged(dec[l], srcs[-1], zb[l], rb, W[l], wl.eps, **kw)
        torch.cuda.synchronize()
        print(f"[merged f24 == merged on decoded] l={l} update={update}", flush=True)
        for a, b, c in zip(r24, r24t, r32):
            assert torch.equal(a, c) and torch.equal(b, c)


@pytest.mark.parametrize("u_format", ["f32", "f24"])
def test_merged_forward_peaked_softmax(u_format):
    """Pseudo-queries ~ N(0, 0.5): scores of std ~40, nearly one-hot weights,
    so the rescaling exp(m - M) often underflows or is exactly 1."""
    for e in _chain(9, 4096, 7168, L=24, w_std=0.5, subs=(0, 23), u_format=u_format):
        assert within_tolerance(e), e
        assert e["alpha_max_abs"] <= TOL_ALPHA_ABS


def test_block_route_full_size_T32768():
    """The bench's block at full size: 8 shared sources and the partial sum,
    24 sub-layers, T = 32768; scores, sums and three sub-layers' merged
    forwards (U sub-layer-major) on every token against the oracle's plain
    forward on all 9 sources, element by element."""
    for e in _chain(9, 32768, 7168, L=24, subs=(0, 11, 23), chunk=4096):
        assert within_tolerance(e), e


def test_block_route_full_size_T32768_f24():
    """The same block with U in the 24-bit format, two sub-layers on every token."""
    for e in _chain(9, 32768, 7168, L=24, subs=(5, 17), chunk=4096, u_format="f24"):
        assert within_tolerance(e), e


def test_merged_agrees_with_scored_and_layouts_bitwise():
    """The merged forward's rstd and alpha agree with the scored forward's: the
    same softmax on the same given scores, only the partial sum's two dots
    summed in another order (fp32 sums of D terms, a few ulps apart; here
    |z| ~ 1, so alpha moves by ~1e-7: 2e-6 leaves a wide margin).  The given
    rstd pass through bitwise, and out, rstd and alpha do not depend on the U
    layout or on the partial sum's row pitch (bitwise)."""
    N, T, D, L = 9, 300, 7168, 24
    wl = synth.workload(1, N=N, T=T)
    bits = wl.sources()
    W = torch.from_numpy(_queries(D, L, 4)).to(DEV)
    srcs = [to_dev_bf16(bits[i]) for i in range(N)]
    rb, zb = ar.attnres_block_scores(srcs[:-1], W, wl.eps)
    U = ar.attnres_block_sums(srcs[:-1], zb)
    Ut = ar.attnres_block_sums(srcs[:-1], zb, token_major=True)
    cache = torch.empty((T, 2, D), dtype=torch.bfloat16, device=DEV)
    cache[:, 1].copy_(srcs[-1])
    for l in (0, 11, 23):
        o_s, r_s, a_s = ar.attnres_fwd_scored(srcs, zb[l], rb, W[l], wl.eps)
        o_m, r_m, a_m = ar.attnres_fwd_merged(U[l], srcs[-1], zb[l], rb, W[l], wl.eps)
        o_t, r_t, a_t = ar.attnres_fwd_merged(Ut[:, l], cache[:, 1], zb[l], rb, W[l], wl.eps)
        torch.cuda.synchronize()
        assert torch.equal(o_t, o_m) and torch.equal(a_t, a_m) and torch.equal(r_t, r_m)
        assert torch.equal(r_m[:, :-1], rb)  # the given rstd pass through
        da = float((a_m - a_s).abs().max())
        dr = float(((r_m - r_s).abs() / r_s).max())
        diff = (o_m.float() - o_s.float()).abs()
        print(f"[merged vs scored] l={l}: alpha max |diff| {da:.3e}, rstd max rel {dr:.3e}, out max |diff| "
              f"{float(diff.max()):.3e}, differing elements {int((diff > 0).sum())} of {o_m.numel()}", flush=True)
        assert da <= 2e-6 and dr <= 2e-6


def test_merged_saved_state_drives_the_backward():
    """The merged forward's saved rstd and alpha, given to the backward with all
    N sources, give the oracle's gradients (every token, element by element)."""
    N, T, D, L = 9, 129, 7168, 24
    wl = synth.workload(1, N=N, T=T)
    bits = wl.sources()
    Wn = _queries(D, L, 5)
    W = torch.from_numpy(Wn).to(DEV)
    srcs = [to_dev_bf16(bits[i]) for i in range(N)]
    g = wl.dout()
    dout = to_dev_bf16(g)
    rb, zb = ar.attnres_block_scores(srcs[:-1], W, wl.eps)
    U = ar.attnres_block_sums(srcs[:-1], zb)
    out, r_m, a_m = ar.attnres_fwd_merged(U[5], srcs[-1], zb[5], rb, W[5], wl.eps)
    d_m, dw_m = ar.attnres_bwd_sources(dout, srcs, W[5], r_m, a_m)
    torch.cuda.synchronize()
    o_out, o_rstd, o_alpha = oracle.fwd(bits, Wn[5], wl.eps)
    o_dsrc, o_dw = oracle.bwd(bits, Wn[5], wl.eps, g)
    acc = Accum(DEV)
    acc.update(bits, g, Wn[5], dict(out=out, rstd=r_m, alpha=a_m, dsrc=torch.stack(d_m)),
               dict(out=o_out, rstd=o_rstd, alpha=o_alpha, dsrc=o_dsrc, merged=True))
    e = acc.result()
    e["dw_rel_l2"] = float(np.linalg.norm(dw_m.cpu().double().numpy() - o_dw) / np.linalg.norm(o_dw))
    print("[merged -> bwd] " + ", ".join(f"{k}={v:.3e}" for k, v in e.items()), flush=True)
    assert within_tolerance(e), e


@pytest.mark.parametrize("in_place", [False, True], ids=["new_buffer", "in_place"])
def test_merged_forward_with_update(in_place):
    """The fused partial-sum update: partial_out = bf16(partial + delta) bit for
    bit as the oracle rounds it; out, rstd and alpha bitwise those of the
    merged forward on the separately updated partial sum, and within the
    bounds of the oracle's plain forward on the updated sources."""
    N, T, D, L, l = 9, 300, 7168, 24, 7
    wl = synth.workload(1, N=N, T=T)
    bits = wl.sources()
    y_h = synth.Workload("merged_y", T=T, N=1, D=D, seed=9, kind="tiny", tiny_scales=(0.3,)).sources()[0]
    W_h = _queries(D, L, 6)
    W = torch.from_numpy(W_h).to(DEV)
    srcs = [to_dev_bf16(bits[i]) for i in range(N)]
    rb, zb = ar.attnres_block_scores(srcs[:-1], W, wl.eps)
    U = ar.attnres_block_sums(srcs[:-1], zb)
    p = srcs[-1].clone()
    out, rstd, alpha, p_new = ar.attnres_fwd_merged(U[l], p, zb[l], rb, W[l], wl.eps, delta=to_dev_bf16(y_h),
                                                    in_place=in_place)
    torch.cuda.synchronize()
    assert (p_new.data_ptr() == p.data_ptr()) == in_place
    o_p = oracle.add_bf16(bits[-1], y_h)
    assert np.array_equal(p_new.cpu().view(torch.int16).numpy().view(np.uint16), o_p)
    e_out, e_rstd, e_alpha = ar.attnres_fwd_merged(U[l], to_dev_bf16(o_p), zb[l], rb, W[l], wl.eps)
    torch.cuda.synchronize()
    assert torch.equal(out, e_out) and torch.equal(rstd, e_rstd) and torch.equal(alpha, e_alpha)
    srcs_h = np.concatenate([bits[:-1], o_p[None]])
    o_out, o_rstd, o_alpha = oracle.fwd(srcs_h, W_h[l], wl.eps)
    acc = Accum(DEV)
    acc.update(srcs_h, None, W_h[l], dict(out=out, rstd=rstd, alpha=alpha),
               dict(out=o_out, rstd=o_rstd, alpha=o_alpha, merged=True))
    e = acc.result()
    print("[merged update] " + ", ".join(f"{k}={v:.3e}" for k, v in e.items()), flush=True)
    assert within_tolerance(e), e


def test_merged_update_refuses_half_an_update():
    D = 64
    z = torch.zeros((4, 2), device=DEV)
    p = torch.zeros((4, D), dtype=torch.bfloat16, device=DEV)
    U = torch.zeros((4, D), device=DEV)
    w = torch.zeros(D, device=DEV)
    with pytest.raises(ValueError):
        ar.attnres_fwd_merged(U, p, z, z, w, 1e-6, partial_out=p)


def test_empty_batch_is_a_no_op():
    D, L = 7168, 4
    srcs = [torch.empty((0, D), dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    z = torch.empty((L, 0, 3), dtype=torch.float32, device=DEV)
    U24 = ar.attnres_block_sums(srcs, z, u_format="f24")
    assert U24.shape == (L, 0, D, 3)
    U = ar.attnres_block_sums(srcs, z)
    assert U.shape == (L, 0, D)
    out, rstd, alpha = ar.attnres_fwd_merged(U[0], torch.empty((0, D), dtype=torch.bfloat16, device=DEV),
                                             torch.empty((0, 3), device=DEV), torch.empty((0, 3), device=DEV),
                                             torch.zeros(D, device=DEV), 1e-6)
    torch.cuda.synchronize()
    assert out.shape == (0, D) and rstd.shape == (0, 4) and alpha.shape == (0, 4)

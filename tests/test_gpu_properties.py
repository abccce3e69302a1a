"""GPU properties that need no oracle: bitwise determinism, batch invariance,
exact special cases, empty batches and error paths through the binding."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_residuals_depth_amd as ar
import synth
from parity import DEV, run_gpu, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ar.library()


def _inputs(wl):
    return (to_dev_bf16(wl.sources()), torch.from_numpy(wl.w()).to(DEV), to_dev_bf16(wl.dout()))


def _bits(t):
    return t.contiguous().view(torch.int16) if t.dtype == torch.bfloat16 else t.contiguous().view(torch.int32)


def test_bitwise_deterministic():
    wl = synth.workload(1)
    src, w, dout = _inputs(wl)
    a = run_gpu(src, w, wl.eps, dout)
    b = run_gpu(src, w, wl.eps, dout)
    for x, y, name in zip(a, b, ["out", "rstd", "alpha", "dsrc", "dw"]):
        assert torch.equal(_bits(x), _bits(y)), f"{name} differs between runs"


def test_batch_invariance():
    """A token's outputs do not depend on the batch around it or its position."""
    small = synth.workload(1, T=128)
    big = synth.workload(1, T=4096)
    s_src, w, s_dout = _inputs(small)
    b_src, _, b_dout = _inputs(big)
    k = 1111  # embed the small batch at an odd offset
    b_src[:, k:k + 128] = s_src
    b_dout[k:k + 128] = s_dout
    so, sr, sa, sd, _ = run_gpu(s_src, w, small.eps, s_dout)
    bo, br, ba, bd, _ = run_gpu(b_src, w, big.eps, b_dout)
    assert torch.equal(_bits(so), _bits(bo[k:k + 128]))
    assert torch.equal(_bits(sr), _bits(br[k:k + 128]))
    assert torch.equal(_bits(sa), _bits(ba[k:k + 128]))
    assert torch.equal(_bits(sd), _bits(bd[:, k:k + 128]))


def test_zero_query_gives_uniform_weights_and_mean():
    wl = synth.workload(1, T=64)
    src, _, dout = _inputs(wl)
    w0 = torch.zeros(wl.D, device=DEV)
    out, rstd, alpha, dsrc, dw = run_gpu(src, w0, wl.eps, dout)
    assert torch.all(alpha == torch.tensor(1.0 / 9.0, dtype=torch.float32))
    mean = src.float().mean(0)
    assert torch.allclose(out.float(), mean, rtol=8e-3, atol=1e-2)
    # z = 0 and w = 0, so each source receives exactly alpha * dout (one fp32 product) before rounding
    ref = (dout.float() * alpha[:, 3:4]).to(torch.bfloat16)
    assert torch.equal(_bits(dsrc[3]), _bits(ref))


def test_identical_sources_reproduce_the_source():
    wl = synth.workload(1, T=96)
    src, w, dout = _inputs(wl)
    same = src[4:5].expand(9, -1, -1).contiguous()
    out, rstd, alpha, dsrc, dw = run_gpu(same, w, wl.eps, dout)
    assert torch.equal(_bits(out), _bits(same[0]))
    assert torch.allclose(alpha.sum(1), torch.ones(96, device=DEV), atol=1e-6)
    assert float(dw.abs().max()) < 1e-3 * float(dout.float().abs().max())


def test_single_source():
    wl = synth.workload(1, T=50, N=1)
    src, w, dout = _inputs(wl)
    out, rstd, alpha, dsrc, dw = run_gpu(src, w, wl.eps, dout)
    assert torch.all(alpha == 1.0)
    assert torch.equal(_bits(out), _bits(src[0]))
    assert torch.equal(_bits(dsrc[0]), _bits(dout))
    assert float(dw.abs().max()) == 0.0


def test_empty_batch():
    D = 7168
    src = torch.empty((9, 0, D), dtype=torch.bfloat16, device=DEV)
    w = torch.randn(D, device=DEV)
    dout = torch.empty((0, D), dtype=torch.bfloat16, device=DEV)
    out, rstd, alpha = ar.attnres_fwd(src, w, 1e-6)
    assert out.shape == (0, D) and rstd.shape == (0, 9)
    dw = torch.full((D,), 7.0, device=DEV)
    dsrc, dw = ar.attnres_bwd(dout, src, w, rstd, alpha, dw=dw)
    torch.cuda.synchronize()
    assert float(dw.abs().max()) == 0.0


def test_errors_raise_and_write_nothing():
    D = 7168
    src = torch.zeros((10, 4, D), dtype=torch.bfloat16, device=DEV)  # N = 10 > 9
    w = torch.zeros(D, device=DEV)
    out = torch.full((4, D), 3.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ar.AttnResError) as ei:
        ar.attnres_fwd(src, w, 1e-6, out=out)
    assert ei.value.code == 1
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
    src9 = torch.zeros((9, 4, D), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ar.AttnResError):
        ar.attnres_fwd(src9, w, float("nan"))
    o, r, a = ar.attnres_fwd(src9, w, 1e-6)
    small_ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(ar.AttnResError) as ei:
        ar.attnres_bwd(torch.zeros((4, D), dtype=torch.bfloat16, device=DEV), src9, w, r, a, workspace=small_ws)
    assert ei.value.code == 2


def test_stream_argument_is_honoured():
    wl = synth.workload(1, T=256)
    src, w, dout = _inputs(wl)
    ref = run_gpu(src, w, wl.eps, dout)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out, rstd, alpha = ar.attnres_fwd(src, w, wl.eps)
        dsrc, dw = ar.attnres_bwd(dout, src, w, rstd, alpha)
    s.synchronize()
    for x, y in zip(ref, (out, rstd, alpha, dsrc, dw)):
        assert torch.equal(_bits(x), _bits(y))


def test_concurrent_calls_on_two_streams():
    """Two host threads, each with its own stream and workload, call fwd + bwd
    three times at once (the library is stateless apart from its
    mutex-guarded occupancy cache, and its kernels do not wait on each
    other): every result equals the same workload run alone, bit for bit."""
    import threading

    cases = [synth.Workload("conc_a", T=700, N=9, D=7168, seed=31), synth.Workload("conc_b", T=333, N=5, D=4096, seed=32)]
    inputs = [_inputs(wl) for wl in cases]
    refs = [run_gpu(src, w, wl.eps, dout) for wl, (src, w, dout) in zip(cases, inputs)]
    torch.cuda.synchronize()
    results = [[None] * 3 for _ in cases]
    errors = []

    def worker(j):
        try:
            wl, (src, w, dout) = cases[j], inputs[j]
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                for k in range(3):
                    out, rstd, alpha = ar.attnres_fwd(src, w, wl.eps)
                    dsrc, dw = ar.attnres_bwd(dout, src, w, rstd, alpha)
                    results[j][k] = (out, rstd, alpha, dsrc, dw)
            s.synchronize()
        except Exception as e:  # surfaced in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(j,)) for j in range(len(cases))]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not errors, errors
    torch.cuda.synchronize()
    for j, ref in enumerate(refs):
        for k in range(3):
            for name, x, y in zip(("out", "rstd", "alpha", "dsrc", "dw"), ref, results[j][k]):
                assert torch.equal(_bits(x), _bits(y)), (cases[j].name, k, name)


@pytest.mark.parametrize("case", ["depth_T300", "two_chunks"])
def test_graph_capture_replays_match_eager(case):
    """fwd, bwd and the decoding forward captured in one HIP graph (the library
    enqueues no memsets and allocates nothing): every replay, with new input
    contents copied in and eager work in between, matches eager calls bit for
    bit -- for a small depth batch, and for a batch whose split backward runs
    two chunks (two split launches, two folds, the ring in use)."""
    if case == "depth_T300":
        wl = synth.workload(1, T=300)
    else:
        wl = synth.Workload("graph_chunks", T=ar.SPLIT_CHUNK_SPANS * ar.SPLIT_TOKENS + 20, N=8, D=1032)
        assert ar.bwd_split(wl.N, wl.D)
    src, w, dout = _inputs(wl)
    N, T, D = src.shape
    s_src, s_dout = src.clone(), dout.clone()
    out = torch.empty((T, D), dtype=torch.bfloat16, device=DEV)
    dec = torch.empty_like(out)
    rstd = torch.empty((T, N), dtype=torch.float32, device=DEV)
    alpha = torch.empty_like(rstd)
    dsrc = torch.empty_like(src)
    dw = torch.empty((D,), dtype=torch.float32, device=DEV)
    ws = torch.empty((ar.workspace_bytes(T, N, D),), dtype=torch.uint8, device=DEV)

    def step():
        ar.attnres_fwd(s_src, w, wl.eps, out=out, rstd=rstd, alpha=alpha)
        ar.attnres_bwd(s_dout, s_src, w, rstd, alpha, dsrc=dsrc, dw=dw, workspace=ws)
        ar.attnres_fwd_decode([s_src[i] for i in range(N)], w, wl.eps, out=dec)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for k in range(3):
        wk = synth.Workload(f"graph_{k}", T=T, N=N, D=D, seed=20 + k, kind=wl.kind)
        src_k, dout_k = to_dev_bf16(wk.sources()), to_dev_bf16(wk.dout())
        s_src.copy_(src_k)
        s_dout.copy_(dout_k)
        graph.replay()
        torch.cuda.synchronize()
        ref = run_gpu(src_k, w, wl.eps, dout_k)  # eager, fresh buffers
        torch.cuda.synchronize()
        for name, x, y in zip(("out", "rstd", "alpha", "dsrc", "dw"), ref, (out, rstd, alpha, dsrc, dw)):
            assert torch.equal(_bits(x), _bits(y)), (k, name)
        assert torch.equal(_bits(ref[0]), _bits(dec)), k


def test_graph_capture_block_route_replays_match_eager():
    """The block-level route (block scores with its query split, block sums in
    both element formats, three merged forwards from the fp32 sums and one
    from the 24-bit ones) captured in one HIP graph: every replay, with new
    sources and queries copied in and eager work in between, matches eager
    calls in fresh buffers bit for bit."""
    n, T, D, L = 8, 300, 7168, 24
    N = n + 1
    s_src = torch.empty((N, T, D), dtype=torch.bfloat16, device=DEV)
    s_W = torch.empty((L, D), dtype=torch.float32, device=DEV)
    rb = torch.empty((T, n), dtype=torch.float32, device=DEV)
    zb = torch.empty((L, T, n), dtype=torch.float32, device=DEV)
    ws = torch.empty((ar.block_scores_workspace_bytes(L, D),), dtype=torch.uint8, device=DEV)
    U = torch.empty((L, T, D), dtype=torch.float32, device=DEV)
    U24 = torch.empty((L, T, D, 3), dtype=torch.uint8, device=DEV)
    subs = (0, 11, 23)
    outs = [(torch.empty((T, D), dtype=torch.bfloat16, device=DEV), torch.empty((T, N), device=DEV),
             torch.empty((T, N), device=DEV)) for _ in range(len(subs) + 1)]
    l24 = 5
    eps = 1e-6

    def step():
        srcs = [s_src[i] for i in range(N)]
        ar.attnres_block_scores(srcs[:n], s_W, eps, rstd=rb, z=zb, workspace=ws)
        ar.attnres_block_sums(srcs[:n], zb, U=U)
        ar.attnres_block_sums(srcs[:n], zb, U=U24, u_format="f24")
        for l, (o, r, a) in zip(subs, outs):
            ar.attnres_fwd_merged(U[l], srcs[n], zb[l], rb, s_W[l], eps, out=o, rstd=r, alpha=a)
        o, r, a = outs[-1]
        ar.attnres_fwd_merged(U24[l24], srcs[n], zb[l24], rb, s_W[l24], eps, out=o, rstd=r, alpha=a)

    def inputs(k):
        wk = synth.Workload(f"graph_block_{k}", T=T, N=N, D=D, seed=40 + k)
        W = np.stack([synth.normal_f32(D, 40 + k, 70 + l, 1.0 / np.sqrt(D)) for l in range(L)])
        return to_dev_bf16(wk.sources()), torch.from_numpy(W).to(DEV)

    src0, W0 = inputs(0)
    s_src.copy_(src0)
    s_W.copy_(W0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for k in range(1, 4):
        src_k, W_k = inputs(k)
        s_src.copy_(src_k)
        s_W.copy_(W_k)
        graph.replay()
        torch.cuda.synchronize()
        srcs = [src_k[i] for i in range(N)]
        r_rb, r_zb = ar.attnres_block_scores(srcs[:n], W_k, eps)  # eager, fresh buffers
        r_U = ar.attnres_block_sums(srcs[:n], r_zb)
        r_U24 = ar.attnres_block_sums(srcs[:n], r_zb, u_format="f24")
        torch.cuda.synchronize()
        assert torch.equal(r_rb, rb) and torch.equal(r_zb, zb) and torch.equal(r_U, U), k
        assert torch.equal(r_U24, U24), k
        for l, (o, r, a), Ue in zip(subs + (l24,), outs, (r_U,) * len(subs) + (r_U24,)):
            e_o, e_r, e_a = ar.attnres_fwd_merged(Ue[l], srcs[n], r_zb[l], r_rb, W_k[l], eps)
            torch.cuda.synchronize()
            assert torch.equal(_bits(e_o), _bits(o)) and torch.equal(e_r, r) and torch.equal(e_a, a), (k, l)

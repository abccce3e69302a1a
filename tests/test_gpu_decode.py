"""The decoding forward (attnres_fwd_decode): per-token results bitwise equal to
the training forward's in any batch, optional saved state, and parity with the
fp64 oracle."""
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


def _inputs(wl):
    src = to_dev_bf16(wl.sources())
    return [src[i] for i in range(wl.N)], torch.from_numpy(wl.w()).to(DEV)


@pytest.mark.parametrize("N,T,D", [(9, 1, 7168), (9, 300, 7168), (9, 1100, 7168), (3, 130, 1000), (5, 40, 12288),
                                   (1, 17, 7168), (2, 5, 16384), (4, 3, 8), (7, 64, 4104)],
                         ids=lambda v: str(v))
def test_decode_equals_training_forward_bitwise(N, T, D):
    wl = synth.Workload(f"dec_N{N}_T{T}_D{D}", T=T, N=N, D=D)
    srcs, w = _inputs(wl)
    o1, r1, a1 = ar.attnres_fwd_sources(srcs, w, wl.eps)
    o2, r2, a2 = ar.attnres_fwd_decode(srcs, w, wl.eps, save_state=True)
    o3, r3, a3 = ar.attnres_fwd_decode(srcs, w, wl.eps)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o1), _bits(o2))
    assert torch.equal(_bits(r1), _bits(r2))
    assert torch.equal(_bits(a1), _bits(a2))
    assert r3 is None and a3 is None
    assert torch.equal(_bits(o1), _bits(o3))


def test_decoding_tokens_one_by_one_matches_the_training_batch():
    """Tokens decoded alone (T = 1) or in a small batch reproduce, bit for bit,
    their rows of a 4096-token training forward."""
    wl = synth.workload(1)  # T = 4096, N = 9, D = 7168
    src = to_dev_bf16(wl.sources())
    w = torch.from_numpy(wl.w()).to(DEV)
    out, rstd, alpha = ar.attnres_fwd(src, w, wl.eps)
    picks = [0, 1, 255, 256, 2047, 4095]
    for t in picks:
        o, r, a = ar.attnres_fwd_decode([src[i, t:t + 1] for i in range(wl.N)], w, wl.eps, save_state=True)
        torch.cuda.synchronize()
        assert torch.equal(_bits(o), _bits(out[t:t + 1])), t
        assert torch.equal(_bits(r), _bits(rstd[t:t + 1])), t
        assert torch.equal(_bits(a), _bits(alpha[t:t + 1])), t
    idx = torch.tensor([4095, 7, 3000, 12, 512, 1999, 64, 65], device=DEV)
    batch = [src[i].index_select(0, idx).contiguous() for i in range(wl.N)]
    o, _, _ = ar.attnres_fwd_decode(batch, w, wl.eps)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o), _bits(out.index_select(0, idx)))


@pytest.mark.parametrize("cfg", [0, 1], ids=["tiny_T128_N3", "depth_T4096_N9"])
def test_decode_against_oracle(cfg):
    wl = synth.workload(cfg, T=min(synth.workload(cfg).T, 512))
    src_h, w_h = wl.sources(), wl.w()
    srcs, w = _inputs(wl)
    out, rstd, alpha = ar.attnres_fwd_decode(srcs, w, wl.eps, save_state=True)
    torch.cuda.synchronize()
    o_out, o_rstd, o_alpha = oracle.fwd(src_h, w_h, wl.eps)
    e_out = rel_l2(bf16_dev_to_f64(out), o_out)
    e_alpha = float(np.max(np.abs(alpha.cpu().double().numpy() - o_alpha)))
    e_rstd = float(np.max(np.abs(rstd.cpu().double().numpy() / o_rstd - 1)))
    print(f"[parity] decode {wl.name} T={wl.T}: out rel_l2={e_out:.3e} alpha max abs={e_alpha:.3e} "
          f"rstd max rel={e_rstd:.3e}", flush=True)
    assert e_out <= TOL_OUT_REL_L2
    assert e_alpha <= TOL_ALPHA_ABS
    assert e_rstd <= TOL_RSTD_REL


def test_decode_empty_batch_is_a_no_op():
    srcs = [torch.empty((0, 7168), dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    w = torch.zeros(7168, device=DEV)
    out, rstd, alpha = ar.attnres_fwd_decode(srcs, w, 1e-6)
    assert out.shape == (0, 7168) and rstd is None and alpha is None

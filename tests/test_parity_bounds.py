"""The element-by-element error bounds the GPU parity tests use (tests/parity.py),
checked on the CPU: an fp32 evaluation of the operator with the kernels' kind
of arithmetic (fp32 sums and products, bf16 round-to-nearest-even of out and
dsources) stays within them on every element of the workloads' distributions,
and a single wrong 16-byte vector (eight channels of one token) breaks them."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import elementwise_ratios, per_token_rel_l2


def _fp32_operator(x_bits, g_bits, w, eps):
    """out, rstd, alpha, dsrc from fp32 arithmetic (sums in torch's own order),
    out and dsrc rounded to bf16: a stand-in for any fp32 implementation."""
    x = torch.from_numpy(synth.bf16_bits_to_f32(x_bits))  # [N][n][D] fp32
    g = torch.from_numpy(synth.bf16_bits_to_f32(g_bits))
    w = torch.from_numpy(w)
    D = x.shape[2]
    r = torch.rsqrt((x * x).sum(2) / D + eps)  # [N][n]
    z = r * (x * w).sum(2)
    a = torch.softmax(z, dim=0)
    out = (a[:, :, None] * x).sum(0).to(torch.bfloat16).double()
    da = (x * g[None]).sum(2)
    s = (a * da).sum(0, keepdim=True)
    c1 = a * (da - s) * r
    k = z * r / D
    dx = a[:, :, None] * g[None] + c1[:, :, None] * (w[None, None, :] - k[:, :, None] * x)
    return (out.numpy(), r.T.contiguous().double().numpy(), a.T.contiguous().double().numpy(),
            dx.to(torch.bfloat16).double().numpy())


@pytest.mark.parametrize("cfg", [1, 3, 4])
def test_fp32_evaluation_within_bounds_and_planted_vector_caught(cfg):
    wl = synth.workload(cfg)
    toks = np.array([0, 1, 2, 77, 1000, 4095], dtype=np.int64)
    x_bits = np.concatenate([wl.sources(int(t), int(t) + 1) for t in toks], axis=1)
    g_bits = np.concatenate([wl.dout(int(t), int(t) + 1) for t in toks], axis=0)
    w = wl.w()
    o_out, o_rstd, o_alpha = oracle.fwd(x_bits, w, wl.eps)
    o_dsrc, _ = oracle.bwd(x_bits, w, wl.eps, g_bits)
    out, rstd, alpha, dsrc = _fp32_operator(x_bits, g_bits, w, wl.eps)
    gpu = dict(out=out, rstd=rstd, alpha=alpha, dsrc=dsrc)
    ref = dict(out=o_out, rstd=o_rstd, alpha=o_alpha, dsrc=o_dsrc)
    e = elementwise_ratios(x_bits, g_bits, w, gpu, ref)
    print(cfg, e, flush=True)
    assert e["out_elem_ratio"] <= 1.0 and e["dsrc_elem_ratio"] <= 1.0, e
    # one wrong 16-byte vector: eight channels of one token take another token's values
    bad_out = out.copy()
    bad_out[3, 800:808] = out[4, 800:808]
    bad_dsrc = dsrc.copy()
    bad_dsrc[wl.N - 1, 2, 8:16] = dsrc[wl.N - 1, 5, 8:16]
    e_bad = elementwise_ratios(x_bits, g_bits, w, dict(gpu, out=bad_out, dsrc=bad_dsrc), ref)
    assert e_bad["out_elem_ratio"] > 10 and e_bad["dsrc_elem_ratio"] > 10, e_bad
    # the whole-tensor relative L2 barely moves, the per-token one does
    assert per_token_rel_l2(bad_out, o_out, 0) > per_token_rel_l2(out, o_out, 0)

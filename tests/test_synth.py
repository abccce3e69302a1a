"""The seeded input generator: reproducible, chunkable, and shaped as stated."""
from __future__ import annotations

import math

import numpy as np
import torch

import synth


def test_rows_are_independent_of_range_and_T():
    wl = synth.workload(1)
    full = wl.with_T(64).sources()
    part = wl.with_T(4096).sources(17, 40)
    assert np.array_equal(full[:, 17:40], part)
    assert np.array_equal(wl.dout(5, 9), wl.with_T(64).dout()[5:9])


def test_deterministic_and_streams_differ():
    wl = synth.workload(0)
    a, b = wl.sources(), wl.sources()
    assert np.array_equal(a, b)
    assert not np.array_equal(a[0], a[1])
    other = synth.Workload("s1", 128, 3, kind="tiny", seed=1)
    assert not np.array_equal(other.sources(), a)


def test_bf16_rounding_matches_torch():
    """The generator's fp32 -> bf16 step is round-to-nearest-even (torch's rule)."""
    n = 1 << 14
    f = synth.normal_f32(n, 0, 77, 3.0)
    bits = synth.rows_bf16(1, n, 0, 77, 0, 3.0)[0]
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)


def test_normal_moments():
    z = synth.normal_f32(1 << 20, 0, 5, 1.0).astype(np.float64)
    assert abs(z.mean()) < 5e-3
    assert abs(z.std() - 1.0) < 5e-3
    assert abs((z ** 4).mean() - 3.0) < 5e-2  # Gaussian kurtosis


def test_depth_scales_and_w():
    wl = synth.workload(1, T=32)
    s = wl.source_scales()
    assert np.allclose(s, np.sqrt(1 + 12 * np.arange(9)), rtol=1e-6)
    x = synth.bf16_bits_to_f32(wl.sources()).astype(np.float64)
    for i in range(9):
        assert abs(x[i].std() / s[i] - 1.0) < 0.02
    w = wl.w().astype(np.float64)
    assert abs(w.std() * math.sqrt(wl.D) - 1.0) < 0.05
    assert abs(synth.workload(3).w().astype(np.float64).std() - 0.5) < 0.02


def test_heavy_workload_structure():
    wl = synth.workload(4, T=16)
    oc = wl.outlier_channels()
    assert len(oc) == 7 and len(set(oc.tolist())) == 7 and oc.min() >= 0 and oc.max() < wl.D
    s = wl.source_scales()
    assert np.all((s[:-1] >= 1.0) & (s[:-1] <= 64.0))
    assert s[-1] == np.float32(1e-4)
    x = synth.bf16_bits_to_f32(wl.sources()).astype(np.float64)
    mask = np.zeros(wl.D, bool)
    mask[oc] = True
    for i in range(wl.N - 1):
        ratio = np.abs(x[i][:, mask]).mean() / np.abs(x[i][:, ~mask]).mean()
        assert 60 < ratio < 160
    last = x[-1]
    assert abs(np.sqrt((last ** 2).mean()) / 1e-4 - 1.0) < 0.05

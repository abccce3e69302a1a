"""Seeded synthetic inputs for the Attention Residuals operator.

This module draws numbers and nothing else: it holds none of the operator's
arithmetic.  Tests, the benchmark and ``__graft_entry__.smoke`` use it to feed
the same bytes to the HIP path (after a host-to-device copy) and to the fp64
oracle.  The C source next to it (``synth.c``) defines the generator; this
wrapper turns the five workloads into tensors.

Workloads (hidden size D = 7168, at most 9 depth sources, as the architecture
figure of "Kimi K3 模型结构（10）：RL 与服务中的状态管理" states; token counts span
the 1K-256K local-token range of the Attention Residuals figure in "Kimi K3 on
Fireworks: Fast RL at frontier scale"):

====  ========  ====  ==========================================  ===============
id    T         N     source i (before bf16 rounding)             w (fp32)
====  ========  ====  ==========================================  ===============
0     128       3     N(0,1) * {1, 2, 4}[i]                       N(0, 1/sqrt(D))
1     4096      9     N(0,1) * sqrt(1 + 12 i)                     N(0, 1/sqrt(D))
2     32768     2..9  as workload 1                               as workload 1
3     131072    9     as workload 1                               N(0, 0.5)
4     262144    9     N(0,1) * 64**u_i, 7 outlier channels x100;  N(0, 1/sqrt(D))
                      last source 1e-4 * N(0,1), no outliers
====  ========  ====  ==========================================  ===============

dout is N(0,1) in bf16 everywhere; eps = 1e-6; seed 0.  N(m, s) names the
standard deviation s.  Every tensor uses its own stream, and element (t, d) of
a [T][D] row set uses counter t * D + d, so token t's inputs do not depend on T
or on which token range is drawn.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")

STREAM_W = 1
STREAM_DOUT = 2
STREAM_SCALE = 3
STREAM_OUTLIER = 4
STREAM_SRC0 = 100  # source i uses stream STREAM_SRC0 + i

D_MODEL = 7168
EPS = 1e-6

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(_LIB_PATH)
        i64, u64, f32 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
        vp = ctypes.c_void_p
        lib.synth_key.argtypes = [u64, u64]
        lib.synth_key.restype = u64
        lib.synth_u64.argtypes = [vp, i64, u64, u64, i64]
        lib.synth_uniform_f64.argtypes = [vp, i64, u64, u64, i64]
        lib.synth_normal_f32.argtypes = [vp, i64, u64, u64, i64, f32]
        lib.synth_rows_bf16.argtypes = [vp, i64, i64, u64, u64, i64, f32, vp]
        for f in (lib.synth_u64, lib.synth_uniform_f64, lib.synth_normal_f32, lib.synth_rows_bf16):
            f.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def u64(n: int, seed: int, stream: int, c0: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().synth_u64(_ptr(out), n, seed, stream, c0)
    return out


def uniform(n: int, seed: int, stream: int, c0: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_uniform_f64(_ptr(out), n, seed, stream, c0)
    return out


def normal_f32(n: int, seed: int, stream: int, scale: float, c0: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _load().synth_normal_f32(_ptr(out), n, seed, stream, c0, float(np.float32(scale)))
    return out


def rows_bf16(rows: int, D: int, seed: int, stream: int, row0: int, scale: float,
              chan_mult: np.ndarray | None = None, out: np.ndarray | None = None) -> np.ndarray:
    """bf16 bit patterns (uint16) of rows row0..row0+rows-1 of a [*][D] stream."""
    if out is None:
        out = np.empty((rows, D), dtype=np.uint16)
    assert out.dtype == np.uint16 and out.shape == (rows, D) and out.flags["C_CONTIGUOUS"]
    cm = None
    if chan_mult is not None:
        chan_mult = np.ascontiguousarray(chan_mult, dtype=np.float32)
        assert chan_mult.shape == (D,)
        cm = _ptr(chan_mult)
    _load().synth_rows_bf16(_ptr(out), rows, D, seed, stream, row0, float(np.float32(scale)), cm)
    return out


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes and value distributions."""

    name: str
    T: int
    N: int
    D: int = D_MODEL
    eps: float = EPS
    seed: int = 0
    kind: str = "depth"  # "tiny" | "depth" | "heavy"
    w_std: float | None = None  # None: 1/sqrt(D)
    tiny_scales: tuple = field(default=(1.0, 2.0, 4.0))

    # -- per-source scales -------------------------------------------------
    def source_scales(self) -> np.ndarray:
        """fp32 scale of each source (before outlier channels)."""
        N = self.N
        if self.kind == "tiny":
            assert N <= len(self.tiny_scales)
            s = np.array(self.tiny_scales[:N], dtype=np.float64)
        elif self.kind == "depth":
            s = np.sqrt(1.0 + 12.0 * np.arange(N, dtype=np.float64))
        elif self.kind == "heavy":
            u = uniform(N, self.seed, STREAM_SCALE)
            s = 64.0 ** u
            s[N - 1] = 1e-4  # near-zero source, exercises eps
        else:
            raise ValueError(self.kind)
        return s.astype(np.float32)

    def outlier_channels(self) -> np.ndarray:
        """Channels multiplied by 100 in every source except the near-zero one."""
        if self.kind != "heavy":
            return np.zeros(0, dtype=np.int64)
        k = int(math.floor(0.001 * self.D))
        chosen: list[int] = []
        c = 0
        while len(chosen) < k:
            d = int(u64(1, self.seed, STREAM_OUTLIER, c)[0] % np.uint64(self.D))
            c += 1
            if d not in chosen:
                chosen.append(d)
        return np.array(sorted(chosen), dtype=np.int64)

    def channel_multipliers(self, i: int) -> np.ndarray | None:
        if self.kind != "heavy" or i == self.N - 1:
            return None
        m = np.ones(self.D, dtype=np.float32)
        m[self.outlier_channels()] = 100.0
        return m

    # -- tensors ---------------------------------------------------------------
    def w(self) -> np.ndarray:
        std = self.w_std if self.w_std is not None else 1.0 / math.sqrt(self.D)
        return normal_f32(self.D, self.seed, STREAM_W, std)

    def sources(self, t0: int = 0, t1: int | None = None, out: np.ndarray | None = None) -> np.ndarray:
        """bf16 bits [N][t1-t0][D] of tokens t0..t1-1."""
        t1 = self.T if t1 is None else t1
        n = t1 - t0
        if out is None:
            out = np.empty((self.N, n, self.D), dtype=np.uint16)
        scales = self.source_scales()
        for i in range(self.N):
            rows_bf16(n, self.D, self.seed, STREAM_SRC0 + i, t0, float(scales[i]),
                      self.channel_multipliers(i), out=out[i])
        return out

    def dout(self, t0: int = 0, t1: int | None = None, out: np.ndarray | None = None) -> np.ndarray:
        """bf16 bits [t1-t0][D] of the output gradient."""
        t1 = self.T if t1 is None else t1
        return rows_bf16(t1 - t0, self.D, self.seed, STREAM_DOUT, t0, 1.0, out=out)

    def with_T(self, T: int) -> "Workload":
        return Workload(self.name, T, self.N, self.D, self.eps, self.seed, self.kind, self.w_std, self.tiny_scales)

    def with_N(self, N: int) -> "Workload":
        return Workload(self.name, self.T, N, self.D, self.eps, self.seed, self.kind, self.w_std, self.tiny_scales)


WORKLOADS = {
    0: Workload("tiny_T128_N3", 128, 3, kind="tiny"),
    1: Workload("depth_T4096_N9", 4096, 9),
    2: Workload("sweep_T32768_N2to9", 32768, 9),
    3: Workload("peaked_T131072_N9", 131072, 9, w_std=0.5),
    4: Workload("heavy_T262144_N9", 262144, 9, kind="heavy"),
}


def workload(i: int, N: int | None = None, T: int | None = None) -> Workload:
    w = WORKLOADS[i]
    if N is not None:
        w = w.with_N(N)
    if T is not None:
        w = w.with_T(T)
    return w


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (a format conversion, not arithmetic of the method)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)

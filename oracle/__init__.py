"""fp64 CPU oracle for the Attention Residuals operator -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never imports it, and the two share no code.

The arithmetic lives in ``attnres_oracle.c`` (plain double-precision loops, one
token at a time).  It follows the formula box of the architecture figure in
"Kimi K3 模型结构（10）：RL 与服务中的状态管理": softmax over the sources of the
pseudo-query w_l dotted with each RMS-normalised source, then the softmax-
weighted sum of the raw sources.  The backward pass is the chain rule of that
formula.  Inputs are the exact bf16 / fp32 values widened to double; outputs
stay in double.

Every function here is pinned by ``tests/test_oracle.py`` against finite
differences, an independent PyTorch fp64 autograd route, hand-derived closed
forms (``tests/golden/``) and invariants of the formula; the partial-sum
update (``add_bf16``) against exact rational arithmetic and hand-worked
rounding cases; the block-batched scores (``block_scores``) against PyTorch's
fp64 ``rms_norm`` and matmul and hand-derived constant-row cases, and the
forward from given scores (``fwd_scored``) against the plain forward and the
two-source sigmoid closed form; the block-batched shared sums (``block_sums``)
and the forward from them (``fwd_merged``) against hand-worked sums, the plain
forward, and the limits where one side of the softmax takes all the weight;
the shared sums' 24-bit storage format (``round24``, ``decode24``) against
hand-worked encodings (ties, carries, subnormals, overflow) and exact rational
rounding.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
MAX_SOURCES = 16

class Oracle:
    """ctypes view of one build of the oracle library (the default one, or a
    deliberately mutated copy that the pin tests compile to prove the pins
    catch mistakes)."""

    def __init__(self, lib_path: str = _LIB_PATH):
        if not os.path.exists(lib_path):
            raise RuntimeError(f"{lib_path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(lib_path)
        i32, i64, f64, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        for name in ("oracle_fwd", "oracle_bwd", "oracle_fwd_f64", "oracle_bwd_f64"):
            f = getattr(lib, name)
            f.argtypes = [i32, i64, i64, vp, vp, f64, vp, vp, vp]
            f.restype = None
        lib.oracle_add_bf16.argtypes = [i64, vp, vp, vp]
        lib.oracle_round24.argtypes = [i64, vp, vp]
        lib.oracle_round24.restype = None
        lib.oracle_decode24.argtypes = [i64, vp, vp]
        lib.oracle_decode24.restype = None
        lib.oracle_add_bf16.restype = None
        lib.oracle_block_scores.argtypes = [i32, i64, i64, i32, vp, vp, f64, vp, vp]
        lib.oracle_block_scores.restype = None
        lib.oracle_fwd_scored.argtypes = [i32, i64, i64, vp, vp, vp, vp, f64, vp, vp, vp]
        lib.oracle_fwd_scored.restype = None
        lib.oracle_block_sums.argtypes = [i32, i64, i64, i32, vp, vp, vp]
        lib.oracle_block_sums.restype = None
        lib.oracle_fwd_merged.argtypes = [i32, i64, i64, vp, vp, vp, vp, vp, f64, vp, vp, vp]
        lib.oracle_fwd_merged.restype = None
        self.lib = lib
        self.path = lib_path

    def add_bf16(self, p_bits: np.ndarray, y_bits: np.ndarray) -> np.ndarray:
        """Partial-sum update: bf16(p + y), rounded once, ties to even (bit patterns in and out)."""
        p_bits = np.ascontiguousarray(p_bits, dtype=np.uint16)
        y_bits = np.ascontiguousarray(y_bits, dtype=np.uint16)
        assert p_bits.shape == y_bits.shape
        out = np.empty_like(p_bits)
        self.lib.oracle_add_bf16(p_bits.size, _p(p_bits), _p(y_bits), _p(out))
        return out

    def round24(self, x: np.ndarray) -> np.ndarray:
        """The 24-bit element format of the block sums: x (float32) rounded to
        16 significant bits, ties to even, kept as the upper three bytes of
        the fp32 pattern; returns uint8 with a trailing dimension of 3."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape + (3,), dtype=np.uint8)
        self.lib.oracle_round24(x.size, _p(x), _p(out))
        return out

    def decode24(self, b: np.ndarray) -> np.ndarray:
        """float32 values of 24-bit elements ([..., 3] uint8)."""
        b = np.ascontiguousarray(b, dtype=np.uint8)
        assert b.shape[-1] == 3
        out = np.empty(b.shape[:-1], dtype=np.float32)
        self.lib.oracle_decode24(out.size, _p(b), _p(out))
        return out

    def fwd_update(self, src_bits: np.ndarray, p_bits: np.ndarray, y_bits: np.ndarray, w: np.ndarray, eps: float):
        """Forward whose last source is the updated partial sum bf16(p + y).

        src_bits: the other N-1 sources [N-1][T][D] (N-1 may be 0); p_bits,
        y_bits: [T][D].  Returns (out, rstd, alpha, p_new bits)."""
        p_new = self.add_bf16(p_bits, y_bits)
        srcs = np.concatenate([np.asarray(src_bits, dtype=np.uint16).reshape(-1, *p_new.shape), p_new[None]], axis=0)
        out, rstd, alpha = self.fwd(srcs, w, eps)
        return out, rstd, alpha, p_new

    def fwd(self, src_bits: np.ndarray, w: np.ndarray, eps: float):
        """Forward on bf16 bit patterns src [N][T][D] (uint16) and fp32 w [D].

        Returns (out [T][D], rstd [T][N], alpha [T][N]) in float64.
        """
        src_bits = np.ascontiguousarray(src_bits, dtype=np.uint16)
        w = np.ascontiguousarray(w, dtype=np.float32)
        N, T, D = _shape(src_bits)
        assert w.shape == (D,)
        out = np.empty((T, D))
        rstd = np.empty((T, N))
        alpha = np.empty((T, N))
        self.lib.oracle_fwd(N, T, D, _p(src_bits), _p(w), float(eps), _p(out), _p(rstd), _p(alpha))
        return out, rstd, alpha

    def bwd(self, src_bits: np.ndarray, w: np.ndarray, eps: float, dout_bits: np.ndarray, want_dsrc: bool = True):
        """Backward on bf16 bit patterns; returns (dsrc [N][T][D] or None, dw [D]) in float64."""
        src_bits = np.ascontiguousarray(src_bits, dtype=np.uint16)
        dout_bits = np.ascontiguousarray(dout_bits, dtype=np.uint16)
        w = np.ascontiguousarray(w, dtype=np.float32)
        N, T, D = _shape(src_bits)
        assert w.shape == (D,) and dout_bits.shape == (T, D)
        dsrc = np.empty((N, T, D)) if want_dsrc else None
        dw = np.empty(D)
        self.lib.oracle_bwd(N, T, D, _p(src_bits), _p(w), float(eps), _p(dout_bits), _p(dsrc), _p(dw))
        return dsrc, dw

    def block_scores(self, src_bits: np.ndarray, W: np.ndarray, eps: float):
        """Block-batched scores: for the n sources src [n][T][D] (bf16 bits) shared
        by the L sub-layers of a block and their pseudo-queries W [L][D] (fp32),
        returns (rstd [T][n], z [L][T][n]) in float64."""
        src_bits = np.ascontiguousarray(src_bits, dtype=np.uint16)
        W = np.ascontiguousarray(W, dtype=np.float32)
        n, T, D = _shape(src_bits)
        L = W.shape[0]
        assert W.shape == (L, D)
        rstd = np.empty((T, n))
        z = np.empty((L, T, n))
        self.lib.oracle_block_scores(n, T, D, L, _p(src_bits), _p(W), float(eps), _p(rstd), _p(z))
        return rstd, z

    def fwd_scored(self, src_bits: np.ndarray, z_given: np.ndarray, r_given: np.ndarray, w: np.ndarray, eps: float):
        """Forward of one sub-layer from given scores: src [N][T][D] bf16 bits (the
        partial sum last), z_given and r_given [T][N-1] for the first N-1
        sources, w [D] fp32 for the last.  Returns (out, rstd [T][N], alpha [T][N])."""
        src_bits = np.ascontiguousarray(src_bits, dtype=np.uint16)
        w = np.ascontiguousarray(w, dtype=np.float32)
        N, T, D = _shape(src_bits)
        z_given = np.ascontiguousarray(z_given, dtype=np.float64).reshape(T, N - 1)
        r_given = np.ascontiguousarray(r_given, dtype=np.float64).reshape(T, N - 1)
        assert w.shape == (D,)
        out = np.empty((T, D))
        rstd = np.empty((T, N))
        alpha = np.empty((T, N))
        self.lib.oracle_fwd_scored(N, T, D, _p(src_bits), _p(z_given), _p(r_given), _p(w), float(eps), _p(out),
                                   _p(rstd), _p(alpha))
        return out, rstd, alpha

    def block_sums(self, src_bits: np.ndarray, z: np.ndarray):
        """Block-batched shared sums: for the n shared sources src [n][T][D] (bf16
        bits) and the block's scores z [L][T][n], returns U [L][T][D] in float64,
        U[l][t] = sum_i exp(z[l][t][i] - max_i z[l][t][i]) x_i[t]."""
        src_bits = np.ascontiguousarray(src_bits, dtype=np.uint16)
        n, T, D = _shape(src_bits)
        z = np.ascontiguousarray(z, dtype=np.float64)
        L = z.shape[0]
        assert z.shape == (L, T, n)
        U = np.empty((L, T, D))
        self.lib.oracle_block_sums(n, T, D, L, _p(src_bits), _p(z), _p(U))
        return U

    def fwd_merged(self, U: np.ndarray, p_bits: np.ndarray, z_given: np.ndarray, r_given: np.ndarray, w: np.ndarray,
                   eps: float):
        """Forward of one sub-layer from its shared sum U [T][D] (float64), the
        partial sum p [T][D] (bf16 bits, the last source), and the given scores
        and rstd [T][N-1] of the shared sources.  Returns (out, rstd [T][N],
        alpha [T][N])."""
        U = np.ascontiguousarray(U, dtype=np.float64)
        p_bits = np.ascontiguousarray(p_bits, dtype=np.uint16)
        w = np.ascontiguousarray(w, dtype=np.float32)
        T, D = p_bits.shape
        assert U.shape == (T, D) and w.shape == (D,)
        z_given = np.ascontiguousarray(z_given, dtype=np.float64).reshape(T, -1)
        N = z_given.shape[1] + 1
        assert 2 <= N <= MAX_SOURCES
        r_given = np.ascontiguousarray(r_given, dtype=np.float64).reshape(T, N - 1)
        out = np.empty((T, D))
        rstd = np.empty((T, N))
        alpha = np.empty((T, N))
        self.lib.oracle_fwd_merged(N, T, D, _p(U), _p(p_bits), _p(z_given), _p(r_given), _p(w), float(eps), _p(out),
                                   _p(rstd), _p(alpha))
        return out, rstd, alpha

    def fwd_f64(self, x: np.ndarray, w: np.ndarray, eps: float):
        """Forward on float64 sources x [N][T][D] and float64 w [D]."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        w = np.ascontiguousarray(w, dtype=np.float64)
        N, T, D = _shape(x)
        assert w.shape == (D,)
        out = np.empty((T, D))
        rstd = np.empty((T, N))
        alpha = np.empty((T, N))
        self.lib.oracle_fwd_f64(N, T, D, _p(x), _p(w), float(eps), _p(out), _p(rstd), _p(alpha))
        return out, rstd, alpha

    def bwd_f64(self, x: np.ndarray, w: np.ndarray, eps: float, g: np.ndarray):
        """Backward on float64 inputs; returns (dx [N][T][D], dw [D])."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        w = np.ascontiguousarray(w, dtype=np.float64)
        g = np.ascontiguousarray(g, dtype=np.float64)
        N, T, D = _shape(x)
        assert w.shape == (D,) and g.shape == (T, D)
        dx = np.empty((N, T, D))
        dw = np.empty(D)
        self.lib.oracle_bwd_f64(N, T, D, _p(x), _p(w), float(eps), _p(g), _p(dx), _p(dw))
        return dx, dw


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _shape(src):
    assert src.ndim == 3, "sources are [N][T][D]"
    N, T, D = src.shape
    assert 1 <= N <= MAX_SOURCES
    return N, T, D


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def fwd(src_bits, w, eps):
    return default().fwd(src_bits, w, eps)


def bwd(src_bits, w, eps, dout_bits, want_dsrc=True):
    return default().bwd(src_bits, w, eps, dout_bits, want_dsrc)


def fwd_f64(x, w, eps):
    return default().fwd_f64(x, w, eps)


def bwd_f64(x, w, eps, g):
    return default().bwd_f64(x, w, eps, g)


def block_scores(src_bits, W, eps):
    return default().block_scores(src_bits, W, eps)


def fwd_scored(src_bits, z_given, r_given, w, eps):
    return default().fwd_scored(src_bits, z_given, r_given, w, eps)


def block_sums(src_bits, z):
    return default().block_sums(src_bits, z)


def fwd_merged(U, p_bits, z_given, r_given, w, eps):
    return default().fwd_merged(U, p_bits, z_given, r_given, w, eps)


def add_bf16(p_bits, y_bits):
    return default().add_bf16(p_bits, y_bits)


def round24(x):
    return default().round24(x)


def decode24(b):
    return default().decode24(b)


def fwd_update(src_bits, p_bits, y_bits, w, eps):
    return default().fwd_update(src_bits, p_bits, y_bits, w, eps)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)

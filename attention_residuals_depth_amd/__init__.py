"""Python binding of libattnres (Attention Residuals forward/backward on MI355X).

Argument marshalling only: every step of the operator runs in the HIP kernels
of ``libattnres.so`` (built from ``csrc/attnres.hip`` for gfx950).  PyTorch
supplies device memory and the stream; outputs are allocated with torch unless
the caller passes them in.  There is no fallback path: if the library is
missing or a call fails, an exception is raised.

The C entry points, declared in ``include/attnres.h``:

    attnres_fwd(src[N][T][D] bf16, w[D] fp32, eps, N, T, D,
                out[T][D] bf16, rstd[T][N] fp32, alpha[T][N] fp32, stream)
    attnres_bwd(dout[T][D] bf16, src, w, rstd, alpha, N, T, D,
                dsrc[N][T][D] bf16, dw[D] fp32, workspace, workspace_bytes, stream)
    attnres_fwd_sources / attnres_bwd_sources: the same with the N sources
                (and their gradients) as separate [T][D] tensors, and an
                accumulate flag for the source gradients.
    attnres_fwd_decode: the per-source forward with rstd/alpha optional
                (decoding / rollout); bitwise the same per-token results as
                the other forward calls.
    attnres_fwd_update: the forward whose last source is the current block's
                partial sum after adding the previous sub-layer's output
                (partial_out = bf16(partial + delta), in place by default).
    attnres_bwd_noalloc: attnres_bwd without a workspace argument, for
                callers that cannot allocate (its dw partial rows live in a
                static device array of the library, D <= 8192).
    attnres_block_scores / attnres_fwd_scored: the rstd and the scores of
                all L pseudo-queries of a block against the sources its
                sub-layers share, in one MFMA pass; then each sub-layer's
                forward from its slice of those scores.
    attnres_block_sums / attnres_fwd_merged: from those scores, the part of
                every sub-layer's weighted sum that the shared sources
                contribute (summed in fp32, before the softmax normaliser;
                stored as fp32 or in the 24-bit format), in one pass; then
                each sub-layer's forward from its shared sum and the partial
                sum alone.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattnres.so")

MAX_SOURCES = 9
MAX_D = 16384
DW_PARTIALS = 256

STATUS = {0: "ATTNRES_OK", 1: "ATTNRES_ERR_INVALID_ARGUMENT", 2: "ATTNRES_ERR_WORKSPACE", 3: "ATTNRES_ERR_HIP"}


class AttnResError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} returned {STATUS.get(code, code)}")
        self.code = code


_lib = None


def library() -> ctypes.CDLL:
    """Load libattnres.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        lib.attnres_fwd.argtypes = [vp, vp, f32, i32, i64, i32, vp, vp, vp, vp]
        lib.attnres_fwd.restype = ctypes.c_int
        lib.attnres_bwd.argtypes = [vp, vp, vp, vp, vp, i32, i64, i32, vp, vp, vp, sz, vp]
        lib.attnres_bwd.restype = ctypes.c_int
        pp = ctypes.POINTER(ctypes.c_void_p)
        lib.attnres_fwd_sources.argtypes = [pp, i64, vp, f32, i32, i64, i32, vp, vp, vp, vp]
        lib.attnres_fwd_sources.restype = ctypes.c_int
        lib.attnres_bwd_sources.argtypes = [vp, pp, i64, vp, vp, vp, i32, i64, i32, pp, i64, i32, vp, vp, sz, vp]
        lib.attnres_bwd_sources.restype = ctypes.c_int
        lib.attnres_fwd_decode.argtypes = [pp, i64, vp, f32, i32, i64, i32, vp, vp, vp, vp]
        lib.attnres_fwd_decode.restype = ctypes.c_int
        lib.attnres_fwd_update.argtypes = [pp, i64, vp, vp, vp, f32, i32, i64, i32, vp, vp, vp, vp, vp]
        lib.attnres_fwd_update.restype = ctypes.c_int
        lib.attnres_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i64, i32, vp, vp, vp]
        lib.attnres_bwd_noalloc.restype = ctypes.c_int
        lib.attnres_block_scores.argtypes = [pp, i64, vp, i32, f32, i32, i64, i32, vp, vp, vp, sz, vp]
        lib.attnres_block_scores.restype = ctypes.c_int
        lib.attnres_fwd_scored.argtypes = [pp, i64, vp, vp, vp, f32, i32, i64, i32, vp, vp, vp, vp]
        lib.attnres_fwd_scored.restype = ctypes.c_int
        lib.attnres_block_sums.argtypes = [pp, i64, vp, i32, i32, i64, i32, vp, i64, i64, i32, vp]
        lib.attnres_block_sums.restype = ctypes.c_int
        lib.attnres_fwd_merged.argtypes = [vp, i64, i32, vp, i64, vp, vp, vp, vp, vp, f32, i32, i64, i32, vp, vp, vp,
                                           vp]
        lib.attnres_fwd_merged.restype = ctypes.c_int
        lib.attnres_set_split_spin.argtypes = [ctypes.c_uint32]
        lib.attnres_set_split_spin.restype = ctypes.c_uint32
        _lib = lib
    return _lib


SPLIT_MAX_D = 7168
SPLIT_ANY_N_MAX_D = 1024
SPLIT_MIN_N = 8
SPLIT_TOKENS = 4
SPLIT_RING = 4096
SPLIT_CHUNK_SPANS = 8192
SPLIT_SPIN_DEFAULT = 4096


def set_split_spin(polls: int) -> int:
    """attnres_set_split_spin: the split backward's poll bound for later calls
    (0 recomputes every member's partial sums); returns the previous bound."""
    if not 0 <= polls < 2**32:
        raise ValueError("polls must fit in 32 bits")
    return int(library().attnres_set_split_spin(polls))


def bwd_split(N: int, D: int) -> bool:
    """ATTNRES_BWD_SPLIT: whether attnres_bwd / attnres_bwd_sources run the split
    backward (else the one-token-per-workgroup backward) for N sources of D."""
    return D <= SPLIT_ANY_N_MAX_D or (N >= SPLIT_MIN_N and D <= SPLIT_MAX_D)


def workspace_bytes(T: int, N: int, D: int) -> int:
    """Bytes of device workspace attnres_bwd / attnres_bwd_sources need
    (ATTNRES_BWD_WORKSPACE_BYTES(T, N, D)): the dw partial rows and, where the
    split backward runs, its exchange ring and one chunk's partial rows."""
    b = DW_PARTIALS * D * 4
    if bwd_split(N, D):
        spans = min((T + SPLIT_TOKENS - 1) // SPLIT_TOKENS, SPLIT_CHUNK_SPANS)
        b += SPLIT_RING * ((D + 1023) // 1024) * 2 * N * 8 + spans * D * 4
    return b


def _stream_handle(stream, dev: torch.device) -> int:
    """The stream to enqueue on: the given one, else the current stream of the
    tensors' device.  The library launches on the current device, so the call
    sites run with `dev` current (see _device)."""
    s = torch.cuda.current_stream(dev) if stream is None else stream
    if s.device != dev:
        raise ValueError(f"stream is on {s.device}, the tensors on {dev}")
    return s.cuda_stream


def _device(dev: torch.device):
    """Make `dev` the current device for the duration of a library call (a
    no-op when it already is)."""
    if dev.index is None or torch.cuda.current_device() == dev.index:
        return contextlib.nullcontext()
    return torch.cuda.device(dev)


def _same_device(dev: torch.device, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev} like the sources")


def _check(t: torch.Tensor, name: str, dtype: torch.dtype, shape: tuple):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def attnres_fwd(src: torch.Tensor, w: torch.Tensor, eps: float, out=None, rstd=None, alpha=None, stream=None):
    """Forward.  src [N][T][D] bf16, w [D] fp32 -> (out [T][D] bf16, rstd [T][N] fp32, alpha [T][N] fp32)."""
    if src.dim() != 3:
        raise ValueError("src must be [N][T][D]")
    N, T, D = src.shape
    _check(src, "src", torch.bfloat16, (N, T, D))
    _check(w, "w", torch.float32, (D,))
    dev = src.device
    if out is None:
        out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    if rstd is None:
        rstd = torch.empty((T, N), dtype=torch.float32, device=dev)
    if alpha is None:
        alpha = torch.empty((T, N), dtype=torch.float32, device=dev)
    _check(out, "out", torch.bfloat16, (T, D))
    _check(rstd, "rstd", torch.float32, (T, N))
    _check(alpha, "alpha", torch.float32, (T, N))
    _same_device(dev, w=w, out=out, rstd=rstd, alpha=alpha)
    with _device(dev):
        code = library().attnres_fwd(src.data_ptr(), w.data_ptr(), float(eps), N, T, D, out.data_ptr(),
                                     rstd.data_ptr(), alpha.data_ptr(), _stream_handle(stream, dev))
    if code != 0:
        raise AttnResError("attnres_fwd", code)
    return out, rstd, alpha


def attnres_bwd(dout: torch.Tensor, src: torch.Tensor, w: torch.Tensor, rstd: torch.Tensor, alpha: torch.Tensor,
                dsrc=None, dw=None, workspace=None, stream=None):
    """Backward.  Returns (dsrc [N][T][D] bf16, dw [D] fp32)."""
    if src.dim() != 3:
        raise ValueError("src must be [N][T][D]")
    N, T, D = src.shape
    _check(src, "src", torch.bfloat16, (N, T, D))
    _check(dout, "dout", torch.bfloat16, (T, D))
    _check(w, "w", torch.float32, (D,))
    _check(rstd, "rstd", torch.float32, (T, N))
    _check(alpha, "alpha", torch.float32, (T, N))
    dev = src.device
    if dsrc is None:
        dsrc = torch.empty((N, T, D), dtype=torch.bfloat16, device=dev)
    if dw is None:
        dw = torch.empty((D,), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty((workspace_bytes(T, N, D),), dtype=torch.uint8, device=dev)
    _check(dsrc, "dsrc", torch.bfloat16, (N, T, D))
    _check(dw, "dw", torch.float32, (D,))
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    _same_device(dev, dout=dout, w=w, rstd=rstd, alpha=alpha, dsrc=dsrc, dw=dw, workspace=workspace)
    with _device(dev):
        code = library().attnres_bwd(dout.data_ptr(), src.data_ptr(), w.data_ptr(), rstd.data_ptr(),
                                     alpha.data_ptr(), N, T, D, dsrc.data_ptr(), dw.data_ptr(), workspace.data_ptr(),
                                     ws_bytes, _stream_handle(stream, dev))
    if code != 0:
        raise AttnResError("attnres_bwd", code)
    return dsrc, dw


NOALLOC_MAX_D = 8192


def attnres_bwd_noalloc(dout: torch.Tensor, src: torch.Tensor, w: torch.Tensor, rstd: torch.Tensor,
                        alpha: torch.Tensor, dsrc: torch.Tensor, dw: torch.Tensor, stream=None):
    """Backward like attnres_bwd, for callers that cannot allocate: no workspace
    (the library keeps the dw partial rows in a static device array, D <= 8192)
    and the outputs must be passed in -- this wrapper allocates nothing either.
    Calls that overlap in time on one device race on that array."""
    if src.dim() != 3:
        raise ValueError("src must be [N][T][D]")
    N, T, D = src.shape
    _check(src, "src", torch.bfloat16, (N, T, D))
    _check(dout, "dout", torch.bfloat16, (T, D))
    _check(w, "w", torch.float32, (D,))
    _check(rstd, "rstd", torch.float32, (T, N))
    _check(alpha, "alpha", torch.float32, (T, N))
    _check(dsrc, "dsrc", torch.bfloat16, (N, T, D))
    _check(dw, "dw", torch.float32, (D,))
    dev = src.device
    _same_device(dev, dout=dout, w=w, rstd=rstd, alpha=alpha, dsrc=dsrc, dw=dw)
    with _device(dev):
        code = library().attnres_bwd_noalloc(dout.data_ptr(), src.data_ptr(), w.data_ptr(), rstd.data_ptr(),
                                             alpha.data_ptr(), N, T, D, dsrc.data_ptr(), dw.data_ptr(),
                                             _stream_handle(stream, dev))
    if code != 0:
        raise AttnResError("attnres_bwd_noalloc", code)
    return dsrc, dw


def _ptr_array(tensors):
    arr = (ctypes.c_void_p * max(1, len(tensors)))()
    for i, t in enumerate(tensors):
        arr[i] = t.data_ptr()
    return arr


def _rows(t: torch.Tensor, name: str, T: int, D: int, dtype=torch.bfloat16) -> int:
    """Check a [T][D] row set whose rows may be spaced apart (a view of one
    source in a token-interleaved [T][N][D] cache); returns its row pitch."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != (T, D):
        raise ValueError(f"{name} must have shape {(T, D)}, got {tuple(t.shape)}")
    if T > 0 and D > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} rows must be contiguous")
    return D if T <= 1 else t.stride(0)


def _sources(srcs, name):
    """Validate N source row sets sharing one row pitch; returns (srcs, T, D, pitch)."""
    srcs = list(srcs)
    if not 1 <= len(srcs) <= MAX_SOURCES:
        raise ValueError(f"{name} must hold 1..{MAX_SOURCES} tensors")
    if not all(isinstance(t, torch.Tensor) for t in srcs):
        raise TypeError(f"{name} must hold torch.Tensor objects")
    if srcs[0].dim() != 2:
        raise ValueError(f"{name}[i] must be [T][D]")
    T, D = srcs[0].shape
    return srcs, T, D, _common_pitch(srcs, name, T, D)


def _common_pitch(tensors, name, T, D, pitch=None, dtype=torch.bfloat16):
    for i, t in enumerate(tensors):
        p = _rows(t, f"{name}[{i}]", T, D, dtype)
        if T > 1:
            if pitch is None:
                pitch = p
            elif p != pitch:
                raise ValueError(f"all of {name} must share one row pitch ({pitch} vs {p})")
    return D if pitch is None else pitch


def attnres_fwd_sources(srcs, w: torch.Tensor, eps: float, out=None, rstd=None, alpha=None, stream=None):
    """Forward on N [T][D] bf16 sources (no stacking copy).  Each source may be
    a separate tensor or a strided view (e.g. cache[:, i, :] of a [T][N][D]
    cache); all must share one row pitch."""
    srcs, T, D, pitch = _sources(srcs, "srcs")
    N = len(srcs)
    _check(w, "w", torch.float32, (D,))
    dev = srcs[0].device
    if out is None:
        out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    if rstd is None:
        rstd = torch.empty((T, N), dtype=torch.float32, device=dev)
    if alpha is None:
        alpha = torch.empty((T, N), dtype=torch.float32, device=dev)
    _check(out, "out", torch.bfloat16, (T, D))
    _check(rstd, "rstd", torch.float32, (T, N))
    _check(alpha, "alpha", torch.float32, (T, N))
    _same_device(dev, w=w, out=out, rstd=rstd, alpha=alpha, **{f"srcs[{i}]": t for i, t in enumerate(srcs)})
    with _device(dev):
        code = library().attnres_fwd_sources(_ptr_array(srcs), pitch, w.data_ptr(), float(eps), N, T, D,
                                             out.data_ptr(), rstd.data_ptr(), alpha.data_ptr(),
                                             _stream_handle(stream, dev))
    if code != 0:
        raise AttnResError("attnres_fwd_sources", code)
    return out, rstd, alpha


def attnres_fwd_decode(srcs, w: torch.Tensor, eps: float, out=None, save_state: bool = False, rstd=None, alpha=None,
                       stream=None):
    """Small-batch forward on N separate [T][D] bf16 sources.  Writes rstd and
    alpha only with save_state=True (or when they are passed).  Returns
    (out, rstd, alpha), the last two None when not saved."""
    srcs, T, D, pitch = _sources(srcs, "srcs")
    N = len(srcs)
    _check(w, "w", torch.float32, (D,))
    dev = srcs[0].device
    if out is None:
        out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, (T, D))
    if save_state or rstd is not None or alpha is not None:
        if rstd is None:
            rstd = torch.empty((T, N), dtype=torch.float32, device=dev)
        if alpha is None:
            alpha = torch.empty((T, N), dtype=torch.float32, device=dev)
        _check(rstd, "rstd", torch.float32, (T, N))
        _check(alpha, "alpha", torch.float32, (T, N))
    _same_device(dev, w=w, out=out, rstd=rstd, alpha=alpha, **{f"srcs[{i}]": t for i, t in enumerate(srcs)})
    with _device(dev):
        code = library().attnres_fwd_decode(_ptr_array(srcs), pitch, w.data_ptr(), float(eps), N, T, D,
                                            out.data_ptr(), None if rstd is None else rstd.data_ptr(),
                                            None if alpha is None else alpha.data_ptr(), _stream_handle(stream, dev))
    if code != 0:
        raise AttnResError("attnres_fwd_decode", code)
    return out, rstd, alpha


def attnres_fwd_update(srcs, partial: torch.Tensor, delta: torch.Tensor, w: torch.Tensor, eps: float,
                       partial_out=None, in_place: bool = True, out=None, save_state: bool = True, rstd=None,
                       alpha=None, stream=None):
    """Forward on the sources srcs (N-1 separate [T][D] bf16 tensors, possibly
    empty) plus the updated partial sum bf16(partial + delta) as the last one.
    The new partial sum goes to partial_out (default: partial itself when
    in_place, else a new tensor).  Returns (out, rstd, alpha, partial_out);
    rstd and alpha are None when save_state is False and none is passed.

    The library writes partial_out behind autograd's back, so the call bumps
    its version counter: an autograd node that saved that tensor (or a view of
    it) then refuses to run its backward instead of reading the updated
    values.  A partial_out that requires grad is refused outright (an
    in-place write into a leaf or a graph tensor)."""
    srcs = list(srcs)
    if partial.dim() != 2:
        raise ValueError("partial must be [T][D]")
    T, D = partial.shape
    N = len(srcs) + 1
    if N > MAX_SOURCES:
        raise ValueError(f"at most {MAX_SOURCES} sources")
    pitch = _common_pitch(srcs + [partial], "srcs+partial", T, D)
    _check(delta, "delta", torch.bfloat16, (T, D))
    _check(w, "w", torch.float32, (D,))
    dev = partial.device
    if partial_out is None:
        if in_place:
            partial_out = partial
        elif pitch == D:
            partial_out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
        else:
            raise ValueError("with strided sources pass partial_out (a row set of the same pitch)")
    _common_pitch([partial_out], "partial_out", T, D, pitch)
    if partial_out.requires_grad:
        raise RuntimeError("partial_out requires grad: the library cannot write it in place under autograd")
    if out is None:
        out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, (T, D))
    if save_state or rstd is not None or alpha is not None:
        if rstd is None:
            rstd = torch.empty((T, N), dtype=torch.float32, device=dev)
        if alpha is None:
            alpha = torch.empty((T, N), dtype=torch.float32, device=dev)
        _check(rstd, "rstd", torch.float32, (T, N))
        _check(alpha, "alpha", torch.float32, (T, N))
    _same_device(dev, delta=delta, w=w, partial_out=partial_out, out=out, rstd=rstd, alpha=alpha,
                 **{f"srcs[{i}]": t for i, t in enumerate(srcs)})
    with _device(dev):
        code = library().attnres_fwd_update(_ptr_array(srcs) if srcs else None, pitch, partial.data_ptr(),
                                            delta.data_ptr(), w.data_ptr(), float(eps), N, T, D,
                                            partial_out.data_ptr(), out.data_ptr(),
                                            None if rstd is None else rstd.data_ptr(),
                                            None if alpha is None else alpha.data_ptr(), _stream_handle(stream, dev))
    if code != 0:
        raise AttnResError("attnres_fwd_update", code)
    torch.autograd.graph.increment_version(partial_out)
    return out, rstd, alpha, partial_out


MAX_QUERIES = 64


def block_scores_workspace_bytes(L: int, D: int) -> int:
    """Bytes of device workspace attnres_block_scores needs (ATTNRES_BLOCK_SCORES_WORKSPACE_BYTES)."""
    return 3 * ((L + 15) // 16 * 16) * ((D + 31) // 32 * 32) * 2


def attnres_block_scores(srcs, W: torch.Tensor, eps: float, rstd=None, z=None, workspace=None, stream=None):
    """Block-batched scores of the n sources a block's sub-layers share (n
    [T][D] bf16 tensors or views with one row pitch) against the block's L
    pseudo-queries W [L][D] fp32: returns (rstd [T][n] fp32, z [L][T][n] fp32),
    z[l] being sub-layer l's scores for attnres_fwd_scored."""
    srcs, T, D, pitch = _sources(srcs, "srcs")
    n = len(srcs)
    if W.dim() != 2:
        raise ValueError("W must be [L][D]")
    L = W.shape[0]
    _check(W, "W", torch.float32, (L, D))
    dev = srcs[0].device
    if rstd is None:
        rstd = torch.empty((T, n), dtype=torch.float32, device=dev)
    if z is None:
        z = torch.empty((L, T, n), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty((block_scores_workspace_bytes(L, D),), dtype=torch.uint8, device=dev)
    _check(rstd, "rstd", torch.float32, (T, n))
    _check(z, "z", torch.float32, (L, T, n))
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    _same_device(dev, W=W, rstd=rstd, z=z, workspace=workspace, **{f"srcs[{i}]": t for i, t in enumerate(srcs)})
    with _device(dev):
        code = library().attnres_block_scores(_ptr_array(srcs), pitch, W.data_ptr(), L, float(eps), n, T, D,
                                              rstd.data_ptr(), z.data_ptr(), workspace.data_ptr(),
                                              workspace.numel() * workspace.element_size(), _stream_handle(stream, dev))
    if code != 0:
        raise AttnResError("attnres_block_scores", code)
    return rstd, z


def attnres_fwd_scored(srcs, z_given: torch.Tensor, rstd_given: torch.Tensor, w: torch.Tensor, eps: float, out=None,
                       rstd=None, alpha=None, stream=None):
    """Forward of one sub-layer from block-batched scores: srcs are the N
    sources, the block's shared ones first and the current partial sum last;
    z_given ([T][N-1], e.g. z[l] of attnres_block_scores) and rstd_given
    ([T][N-1]) are the shared sources' scores and rstd; w [D] scores the
    partial sum.  Returns (out, rstd [T][N], alpha [T][N]) like
    attnres_fwd_sources."""
    srcs, T, D, pitch = _sources(srcs, "srcs")
    N = len(srcs)
    if N < 2:
        raise ValueError("the scored forward needs the shared sources and the partial sum (N >= 2)")
    _check(z_given, "z_given", torch.float32, (T, N - 1))
    _check(rstd_given, "rstd_given", torch.float32, (T, N - 1))
    _check(w, "w", torch.float32, (D,))
    dev = srcs[0].device
    if out is None:
        out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    if rstd is None:
        rstd = torch.empty((T, N), dtype=torch.float32, device=dev)
    if alpha is None:
        alpha = torch.empty((T, N), dtype=torch.float32, device=dev)
    _check(out, "out", torch.bfloat16, (T, D))
    _check(rstd, "rstd", torch.float32, (T, N))
    _check(alpha, "alpha", torch.float32, (T, N))
    _same_device(dev, z_given=z_given, rstd_given=rstd_given, w=w, out=out, rstd=rstd, alpha=alpha,
                 **{f"srcs[{i}]": t for i, t in enumerate(srcs)})
    with _device(dev):
        code = library().attnres_fwd_scored(_ptr_array(srcs), pitch, z_given.data_ptr(), rstd_given.data_ptr(),
                                            w.data_ptr(), float(eps), N, T, D, out.data_ptr(), rstd.data_ptr(),
                                            alpha.data_ptr(), _stream_handle(stream, dev))
    if code != 0:
        raise AttnResError("attnres_fwd_scored", code)
    return out, rstd, alpha


U_F32 = 0  # element formats of the block sums (ATTNRES_U_F32, ATTNRES_U_F24)
U_F24 = 1
_U_FORMATS = {"f32": U_F32, "f24": U_F24}


def decode_u24(U: torch.Tensor) -> torch.Tensor:
    """The fp32 values of block sums stored in the 24-bit format (a uint8
    tensor whose last dimension holds an element's three bytes).  A plain
    torch view for inspection; attnres_fwd_merged reads the format itself."""
    if U.dtype != torch.uint8 or U.dim() < 1 or U.shape[-1] != 3:
        raise ValueError("U must be a uint8 tensor with three bytes per element in its last dimension")
    b = U.to(torch.int64)
    bits = (b[..., 0] << 8) | (b[..., 1] << 16) | (b[..., 2] << 24)  # the fp32 bit pattern, 0 .. 2^32 - 1
    return torch.where(bits >= 2 ** 31, bits - 2 ** 32, bits).to(torch.int32).view(torch.float32)


def attnres_block_sums(srcs, z: torch.Tensor, U=None, token_major: bool = False, u_format: str = "f32",
                       stream=None):
    """Block-batched shared sums of the n sources a block's sub-layers share (n
    [T][D] bf16 tensors or views with one row pitch), from the block's scores z
    [L][T][n] fp32 (attnres_block_scores): U[l][t] = sum_i exp(z[l][t][i] -
    max_i z[l][t][i]) srcs[i][t], summed in fp32.  Returns U as [L][T][D], or
    as [T][L][D] with token_major (sub-layer l's rows are then U[:, l]); a
    given U must have that shape and be contiguous.  u_format "f32" stores
    fp32; "f24" stores each sum rounded to a 16-bit significand in three bytes
    (ATTNRES_U_F24), as a uint8 tensor with one more dimension of 3."""
    if u_format not in _U_FORMATS:
        raise ValueError(f"u_format must be one of {sorted(_U_FORMATS)}")
    fmt = _U_FORMATS[u_format]
    srcs, T, D, pitch = _sources(srcs, "srcs")
    n = len(srcs)
    if z.dim() != 3:
        raise ValueError("z must be [L][T][n]")
    L = z.shape[0]
    _check(z, "z", torch.float32, (L, T, n))
    dev = srcs[0].device
    shape = (T, L, D) if token_major else (L, T, D)
    dtype = torch.float32
    if fmt == U_F24:
        shape, dtype = shape + (3,), torch.uint8
    if U is None:
        U = torch.empty(shape, dtype=dtype, device=dev)
    _check(U, "U", dtype, shape)
    lstride, tpitch = (D, L * D) if token_major else (T * D, D)
    _same_device(dev, z=z, U=U, **{f"srcs[{i}]": t for i, t in enumerate(srcs)})
    with _device(dev):
        code = library().attnres_block_sums(_ptr_array(srcs), pitch, z.data_ptr(), L, n, T, D, U.data_ptr(), lstride,
                                            tpitch, fmt, _stream_handle(stream, dev))
    if code != 0:
        raise AttnResError("attnres_block_sums", code)
    return U


def attnres_fwd_merged(U_l: torch.Tensor, partial: torch.Tensor, z_given: torch.Tensor, rstd_given: torch.Tensor,
                       w: torch.Tensor, eps: float, delta=None, partial_out=None, in_place: bool = True, out=None,
                       rstd=None, alpha=None, stream=None):
    """Forward of one sub-layer from its block-batched shared sum: U_l [T][D]
    fp32, or [T][D][3] uint8 in the 24-bit format (U[l] or U[:, l] of
    attnres_block_sums; rows may be spaced apart),
    partial [T][D] bf16 the current partial sum (the last of the N sources),
    z_given and rstd_given [T][N-1] the shared sources' scores for this
    sub-layer and their rstd (attnres_block_scores).  With delta ([T][D] bf16,
    the previous sub-layer's output) the partial sum is first updated to
    bf16(partial + delta), written to partial_out (default: partial itself
    when in_place, else a new tensor) and used as the last source, as in
    attnres_fwd_update.  Returns (out, rstd [T][N], alpha [T][N]), plus
    partial_out when delta is given."""
    if not isinstance(z_given, torch.Tensor) or z_given.dim() != 2:
        raise ValueError("z_given must be a [T][N-1] tensor")
    T, n = z_given.shape
    N = n + 1
    if not 2 <= N <= MAX_SOURCES:
        raise ValueError(f"N = {N} sources: the merged forward takes 2..{MAX_SOURCES}")
    if not isinstance(partial, torch.Tensor) or partial.dim() != 2:
        raise ValueError("partial must be [T][D]")
    D = partial.shape[1]
    p_pitch = _rows(partial, "partial", T, D)
    if isinstance(U_l, torch.Tensor) and U_l.dtype == torch.uint8:
        fmt = U_F24
        if U_l.device.type != "cuda":
            raise ValueError("U_l must be a device tensor")
        if tuple(U_l.shape) != (T, D, 3):
            raise ValueError(f"a 24-bit U_l must have shape {(T, D, 3)}, got {tuple(U_l.shape)}")
        if T > 0 and D > 0 and (U_l.stride(2) != 1 or (D > 1 and U_l.stride(1) != 3)):
            raise ValueError("U_l rows must be contiguous, three bytes per element")
        if T > 1 and U_l.stride(0) % 3 != 0:
            raise ValueError("U_l rows must start on element boundaries")
        u_pitch = U_l.stride(0) // 3 if T > 1 else D
    else:
        fmt = U_F32
        u_pitch = _rows(U_l, "U_l", T, D, torch.float32)
    _check(z_given, "z_given", torch.float32, (T, N - 1))
    _check(rstd_given, "rstd_given", torch.float32, (T, N - 1))
    _check(w, "w", torch.float32, (D,))
    dev = partial.device
    if delta is not None:
        _check(delta, "delta", torch.bfloat16, (T, D))
        if partial_out is None:
            if in_place:
                partial_out = partial
            elif p_pitch == D:
                partial_out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
            else:
                raise ValueError("with a strided partial sum pass partial_out (a row set of the same pitch)")
        _common_pitch([partial_out], "partial_out", T, D, p_pitch)
        if partial_out.requires_grad:
            raise RuntimeError("partial_out requires grad: the library cannot write it in place under autograd")
    elif partial_out is not None:
        raise ValueError("partial_out is only written with a delta")
    if out is None:
        out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    if rstd is None:
        rstd = torch.empty((T, N), dtype=torch.float32, device=dev)
    if alpha is None:
        alpha = torch.empty((T, N), dtype=torch.float32, device=dev)
    _check(out, "out", torch.bfloat16, (T, D))
    _check(rstd, "rstd", torch.float32, (T, N))
    _check(alpha, "alpha", torch.float32, (T, N))
    _same_device(dev, U_l=U_l, z_given=z_given, rstd_given=rstd_given, w=w, out=out, rstd=rstd, alpha=alpha,
                 **({} if delta is None else {"delta": delta, "partial_out": partial_out}))
    with _device(dev):
        code = library().attnres_fwd_merged(U_l.data_ptr(), u_pitch, fmt, partial.data_ptr(), p_pitch,
                                            None if delta is None else delta.data_ptr(),
                                            None if delta is None else partial_out.data_ptr(), z_given.data_ptr(),
                                            rstd_given.data_ptr(), w.data_ptr(), float(eps), N, T, D, out.data_ptr(),
                                            rstd.data_ptr(), alpha.data_ptr(), _stream_handle(stream, dev))
    if code != 0:
        raise AttnResError("attnres_fwd_merged", code)
    if delta is None:
        return out, rstd, alpha
    torch.autograd.graph.increment_version(partial_out)
    return out, rstd, alpha, partial_out


GRAD_ACCUMULATE = 1  # grad_mode bits of attnres_bwd_sources
GRAD_F32 = 2


def attnres_bwd_sources(dout: torch.Tensor, srcs, w: torch.Tensor, rstd: torch.Tensor, alpha: torch.Tensor,
                        dsrcs=None, accumulate: bool = False, grad_dtype=None, dw=None, workspace=None, stream=None):
    """Backward on N separate sources.  dsrcs: N [T][D] gradient tensors, all
    bf16 or all fp32 (allocated if None, as grad_dtype, default bf16); with
    accumulate=True the new gradients are added to their contents (in fp32,
    then rounded once for bf16).  Sources and gradients may be strided views
    (one row pitch for the sources, one for the gradients).  Returns (dsrcs, dw)."""
    srcs, T, D, pitch = _sources(srcs, "srcs")
    N = len(srcs)
    _check(dout, "dout", torch.bfloat16, (T, D))
    _check(w, "w", torch.float32, (D,))
    _check(rstd, "rstd", torch.float32, (T, N))
    _check(alpha, "alpha", torch.float32, (T, N))
    dev = srcs[0].device
    if dsrcs is None:
        if accumulate:
            raise ValueError("accumulate=True needs the gradient tensors to add to")
        gdt = torch.bfloat16 if grad_dtype is None else grad_dtype
        dsrcs = [torch.empty((T, D), dtype=gdt, device=dev) for _ in range(N)]
    dsrcs = list(dsrcs)
    if len(dsrcs) != N:
        raise ValueError("dsrcs must hold one tensor per source")
    gdt = dsrcs[0].dtype if isinstance(dsrcs[0], torch.Tensor) else torch.bfloat16
    if gdt not in (torch.bfloat16, torch.float32) or (grad_dtype is not None and grad_dtype != gdt):
        raise TypeError(f"gradients must all be torch.bfloat16 or all torch.float32 (got {gdt})")
    dpitch = _common_pitch(dsrcs, "dsrcs", T, D, dtype=gdt)
    mode = (GRAD_ACCUMULATE if accumulate else 0) | (GRAD_F32 if gdt == torch.float32 else 0)
    if dw is None:
        dw = torch.empty((D,), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty((workspace_bytes(T, N, D),), dtype=torch.uint8, device=dev)
    _check(dw, "dw", torch.float32, (D,))
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    _same_device(dev, dout=dout, w=w, rstd=rstd, alpha=alpha, dw=dw, workspace=workspace,
                 **{f"srcs[{i}]": t for i, t in enumerate(srcs)}, **{f"dsrcs[{i}]": t for i, t in enumerate(dsrcs)})
    with _device(dev):
        code = library().attnres_bwd_sources(dout.data_ptr(), _ptr_array(srcs), pitch, w.data_ptr(),
                                             rstd.data_ptr(), alpha.data_ptr(), N, T, D, _ptr_array(dsrcs), dpitch,
                                             mode, dw.data_ptr(), workspace.data_ptr(), ws_bytes,
                                             _stream_handle(stream, dev))
    if code != 0:
        raise AttnResError("attnres_bwd_sources", code)
    return dsrcs, dw


class _AttnResFunction(torch.autograd.Function):
    """Autograd node of one operator call on N separate sources: the forward
    runs attnres_fwd_sources and saves rstd and alpha, the backward runs
    attnres_bwd_sources and returns the gradient of w (fp32) and of every
    source (bf16; autograd adds it to whatever the source's other uses give)."""

    @staticmethod
    def forward(ctx, w, eps, *srcs):
        out, rstd, alpha = attnres_fwd_sources(list(srcs), w, eps)
        ctx.save_for_backward(w, rstd, alpha, *srcs)
        return out

    @staticmethod
    def backward(ctx, dout):
        w, rstd, alpha, *srcs = ctx.saved_tensors
        dout = dout.to(torch.bfloat16).contiguous()  # the backward takes dout in bf16
        dsrcs, dw = attnres_bwd_sources(dout, srcs, w, rstd, alpha)
        return (dw, None, *dsrcs)


def attnres(srcs, w: torch.Tensor, eps: float) -> torch.Tensor:
    """Differentiable call for training code: out [T][D] bf16 from the N
    sources (bf16 [T][D] tensors or views with one common row pitch, e.g.
    slices of a [T][N][D] cache) and w [D] fp32.  Gradients flow to every
    source and to w through the library's backward."""
    return _AttnResFunction.apply(w, float(eps), *_sources(srcs, "srcs")[0])


__all__ = ["attnres", "attnres_fwd", "attnres_bwd", "attnres_fwd_sources", "attnres_bwd_sources", "attnres_fwd_decode",
           "attnres_fwd_update", "attnres_bwd_noalloc", "attnres_block_scores", "attnres_fwd_scored",
           "attnres_block_sums", "attnres_fwd_merged", "U_F32", "U_F24", "decode_u24", "block_scores_workspace_bytes", "MAX_QUERIES", "GRAD_ACCUMULATE", "GRAD_F32", "NOALLOC_MAX_D",
           "SPLIT_MAX_D", "SPLIT_ANY_N_MAX_D", "SPLIT_MIN_N", "bwd_split", "SPLIT_TOKENS", "SPLIT_RING", "SPLIT_CHUNK_SPANS", "SPLIT_SPIN_DEFAULT", "set_split_spin",
           "workspace_bytes", "library", "AttnResError", "MAX_SOURCES", "MAX_D", "DW_PARTIALS", "LIB_PATH"]

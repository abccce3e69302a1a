"""The C ABI without a GPU: the library loads, exports what include/attnres.h
declares, agrees with the binding's constants, and rejects bad arguments on the
host before any HIP call (every call here has at least one invalid argument,
so no device work is ever attempted)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import attention_residuals_depth_amd as ar

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attnres.h")

OK, INVALID, WORKSPACE, HIP = 0, 1, 2, 3
D = 7168
A = 1 << 20  # fake, 16-byte aligned "device addresses"; never dereferenced


def _declared():
    text = open(HEADER).read()
    return re.findall(r"^attnres_status\s+(attnres_\w+)\s*\(", text, re.M)


def _define(name):
    m = re.search(rf"#define\s+{name}\s+(\d+)", open(HEADER).read())
    return int(m.group(1))


def test_library_loads_and_exports_declared_symbols():
    lib = ar.library()
    names = _declared()
    assert names == ["attnres_fwd", "attnres_bwd", "attnres_fwd_sources", "attnres_fwd_decode",
                     "attnres_fwd_update", "attnres_bwd_sources", "attnres_block_scores", "attnres_fwd_scored",
                     "attnres_block_sums", "attnres_fwd_merged", "attnres_bwd_noalloc"]
    others = re.findall(r"^uint32_t\s+(attnres_\w+)\s*\(", open(HEADER).read(), re.M)
    assert others == ["attnres_set_split_spin"]
    names += others
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", ar.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported
    assert not any(s.startswith("oracle_") for s in exported), "the product library must not carry oracle code"


def test_library_is_built_for_gfx950():
    # the offload bundle of a library built here names its target triple
    blob = open(ar.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def test_block_scores_refuses_on_the_host():
    """attnres_block_scores / attnres_fwd_scored: every call below has one bad
    argument and returns its status before anything reaches the GPU."""
    lib = ar.library()
    g = 1 << 30
    srcs = (ctypes.c_void_p * 9)(*[(i + 1) * g for i in range(9)])
    ws = ar.block_scores_workspace_bytes(24, D)

    def blk(n=8, T=16, D_=D, L=24, W=20 * g, eps=1e-6, rstd=21 * g, z=22 * g, w_=23 * g, wsb=None, pitch=None,
            s=srcs):
        return lib.attnres_block_scores(s, D_ if pitch is None else pitch, W, L, eps, n, T, D_, rstd, z, w_,
                                        ws if wsb is None else wsb, None)

    assert _define("ATTNRES_MAX_QUERIES") == ar.MAX_QUERIES == 64
    assert blk(L=0) == INVALID and blk(L=65) == INVALID
    assert blk(n=0) == INVALID and blk(n=10) == INVALID
    assert blk(D_=7170) == INVALID and blk(eps=-1.0) == INVALID and blk(eps=float("nan")) == INVALID
    assert blk(W=20 * g + 4) == INVALID                    # W not 16-byte aligned
    assert blk(rstd=0) == INVALID and blk(z=21 * g + 2) == INVALID
    assert blk(wsb=ws - 16) == WORKSPACE and blk(w_=0) == WORKSPACE
    assert blk(z=1 * g) == INVALID                         # z overlaps source 0
    assert blk(rstd=20 * g) == INVALID                     # rstd overlaps W
    assert blk(pitch=D - 8) == INVALID and blk(pitch=(1 << 24) + 8) == INVALID
    assert blk(T=0, s=None, rstd=0, z=0, w_=0) == OK       # empty: nothing to do

    def scored(N=9, T=16, D_=D, zg=30 * g, rg=31 * g, w=32 * g, out=33 * g, rstd=34 * g, alpha=35 * g):
        return lib.attnres_fwd_scored(srcs, D_, zg, rg, w, 1e-6, N, T, D_, out, rstd, alpha, None)

    assert scored(N=1) == INVALID                          # no shared source
    assert scored(zg=0) == INVALID and scored(rg=0) == INVALID
    assert scored(zg=30 * g + 2) == INVALID                # misaligned
    assert scored(out=30 * g) == INVALID                   # out overlaps the given scores
    assert scored(rstd=31 * g) == INVALID                  # rstd overlaps the given rstd


def test_block_sums_and_merged_forward_refuse_on_the_host():
    """attnres_block_sums / attnres_fwd_merged: every call below has one bad
    argument (or, last, nothing to do) and returns its status before anything
    reaches the GPU."""
    lib = ar.library()
    g = 1 << 30
    srcs = (ctypes.c_void_p * 9)(*[(i + 1) * g for i in range(9)])
    T_, L_ = 16, 24

    def sums(n=8, T=T_, D_=D, L=L_, z=20 * g, U=21 * g, ls=None, tp=None, pitch=None, s=srcs, fmt=ar.U_F32):
        ls = T * D_ if ls is None else ls
        tp = D_ if tp is None else tp
        return lib.attnres_block_sums(s, D_ if pitch is None else pitch, z, L, n, T, D_, U, ls, tp, fmt, None)

    assert sums(L=0) == INVALID and sums(L=65) == INVALID
    assert sums(n=0) == INVALID and sums(n=10) == INVALID
    assert sums(D_=7170) == INVALID and sums(pitch=D - 8) == INVALID
    assert sums(z=0) == INVALID and sums(U=0) == INVALID
    assert sums(z=20 * g + 2) == INVALID and sums(U=21 * g + 8) == INVALID   # misaligned
    assert sums(ls=D, tp=D) == INVALID                     # rows of one sub-layer's tokens would collide
    assert sums(ls=T_ * D - 4, tp=D) == INVALID            # sub-layer-major, one float short
    assert sums(ls=D, tp=(L_ - 1) * D + D - 4) == INVALID  # token-major, one float short
    assert sums(ls=T_ * D + 2) == INVALID                  # not a multiple of 4 floats
    assert sums(tp=D - 4, ls=T_ * D) == INVALID            # pitch below a row
    assert sums(U=1 * g) == INVALID                        # U overlaps source 0
    assert sums(U=20 * g - 1024) == INVALID                # U runs into z
    assert sums(fmt=2) == INVALID and sums(fmt=-1) == INVALID  # no such element format
    assert sums(fmt=ar.U_F24, U=21 * g + 2) == INVALID     # 24-bit elements: a 4-byte aligned base
    # the 24-bit rows span 3 bytes per element: a U whose last 12 bytes lie on z overlaps it
    span24 = ((L_ - 1) * T_ * D + (T_ - 1) * D + D) * 3
    assert sums(fmt=ar.U_F24, U=20 * g - span24 + 12) == INVALID
    assert sums(T=0, s=None, z=0, U=0) == OK               # empty: nothing to do

    def merged(N=9, T=T_, D_=D, U=40 * g, up=None, p=41 * g, pp=None, zg=42 * g, rg=43 * g, w=44 * g, eps=1e-6,
               out=45 * g, rstd=46 * g, alpha=47 * g, y=None, po=None, fmt=ar.U_F32):
        return lib.attnres_fwd_merged(U, D_ if up is None else up, fmt, p, D_ if pp is None else pp, y, po, zg, rg, w,
                                      eps, N, T, D_, out, rstd, alpha, None)

    assert merged(N=1) == INVALID and merged(N=10) == INVALID
    assert merged(U=0) == INVALID and merged(p=0) == INVALID and merged(zg=0) == INVALID and merged(rg=0) == INVALID
    assert merged(out=0) == INVALID and merged(rstd=0) == INVALID and merged(alpha=0) == INVALID
    assert merged(w=0) == INVALID and merged(eps=-1.0) == INVALID and merged(D_=7170) == INVALID
    assert merged(U=40 * g + 8) == INVALID and merged(p=41 * g + 2) == INVALID    # misaligned
    assert merged(up=D - 4) == INVALID and merged(up=D + 2) == INVALID and merged(pp=D + 4) == INVALID
    assert merged(out=40 * g) == INVALID                   # out overlaps U
    assert merged(rstd=42 * g) == INVALID                  # rstd overlaps the given scores
    assert merged(alpha=46 * g) == INVALID                 # alpha overlaps rstd
    assert merged(y=48 * g) == INVALID and merged(po=49 * g) == INVALID  # the update needs both
    assert merged(y=48 * g + 4, po=49 * g) == INVALID                     # misaligned delta
    assert merged(y=48 * g, po=48 * g) == INVALID                         # partial_out on top of delta
    assert merged(y=48 * g, po=40 * g) == INVALID                         # partial_out on top of U
    assert merged(y=48 * g, po=45 * g) == INVALID                         # partial_out on top of out
    assert merged(fmt=2) == INVALID and merged(fmt=ar.U_F24, U=40 * g + 2) == INVALID
    assert merged(fmt=ar.U_F24, out=40 * g + T_ * D * 3 - 16) == INVALID  # out overlaps the last 24-bit U row
    assert merged(T=0, U=0, p=0, zg=0, rg=0, out=0, rstd=0, alpha=0) == OK


def test_header_constants_match_binding():
    assert _define("ATTNRES_NOALLOC_MAX_D") == ar.NOALLOC_MAX_D == 8192
    assert _define("ATTNRES_MAX_SOURCES") == ar.MAX_SOURCES == 9
    assert _define("ATTNRES_MAX_D") == ar.MAX_D
    assert _define("ATTNRES_DW_PARTIALS") == ar.DW_PARTIALS
    assert _define("ATTNRES_U_F32") == ar.U_F32 == 0 and _define("ATTNRES_U_F24") == ar.U_F24 == 1
    for name in ("SPLIT_MAX_D", "SPLIT_ANY_N_MAX_D", "SPLIT_MIN_N", "SPLIT_TOKENS", "SPLIT_RING", "SPLIT_CHUNK_SPANS",
                 "SPLIT_SPIN_DEFAULT"):
        assert _define("ATTNRES_" + name) == getattr(ar, name)
    # the split backward where it measured faster: every N up to D = 1024, N >= 8 up to D = 7168
    assert ar.bwd_split(1, 8) and ar.bwd_split(3, 1024) and ar.bwd_split(8, 7168) and ar.bwd_split(9, 2048)
    assert not ar.bwd_split(7, 7168) and not ar.bwd_split(9, 7176) and not ar.bwd_split(2, 1032)
    # the backward's workspace: 256 partial rows, and where the split backward runs the exchange
    # ring (4096 tokens x ceil(D/1024) slices x 2N words of 8 bytes) and the
    # partial rows of one chunk of spans (ceil(T/4) rows, at most 8192): 32768
    # tokens and above need the same
    assert ar.workspace_bytes(131072, 9, D) == 256 * D * 4 + 4096 * 7 * 18 * 8 + 8192 * D * 4 == 246_349_824
    assert ar.workspace_bytes(32768, 9, D) == ar.workspace_bytes(131072, 9, D) == ar.workspace_bytes(262144, 9, D)
    assert ar.workspace_bytes(32764, 9, D) == 256 * D * 4 + 4096 * 7 * 18 * 8 + 8191 * D * 4
    assert ar.workspace_bytes(1, 1, 8) == 256 * 8 * 4 + 4096 * 1 * 2 * 8 + 8 * 4
    assert ar.workspace_bytes(1000, 9, 12288) == 256 * 12288 * 4  # one-token-per-workgroup backward
    assert ar.workspace_bytes(131072, 7, D) == 256 * D * 4  # one-token backward for N <= 7 at D = 7168


def _fwd(src=A, w=2 * A, eps=1e-6, N=9, T=16, D_=D, out=None, rstd=None, alpha=None):
    base = 1 << 36
    out = base if out is None else out
    rstd = base + (1 << 30) if rstd is None else rstd
    alpha = base + (1 << 31) if alpha is None else alpha
    return ar.library().attnres_fwd(src, w, eps, N, T, D_, out, rstd, alpha, None)


def _bwd(dout=None, src=None, w=None, rstd=None, alpha=None, N=9, T=16, D_=D, dsrc=None, dw=None, ws=None,
         ws_bytes=None):
    g = 1 << 30
    vals = dict(dout=1 * g, src=2 * g, w=3 * g, rstd=4 * g, alpha=5 * g, dsrc=8 * g, dw=12 * g, ws=13 * g)
    for k, v in dict(dout=dout, src=src, w=w, rstd=rstd, alpha=alpha, dsrc=dsrc, dw=dw, ws=ws).items():
        if v is not None:
            vals[k] = v
    if ws_bytes is None:
        ws_bytes = ar.workspace_bytes(T, max(N, 1), D_)
    return ar.library().attnres_bwd(vals["dout"], vals["src"], vals["w"], vals["rstd"], vals["alpha"], N, T, D_,
                                    vals["dsrc"], vals["dw"], vals["ws"], ws_bytes, None)


@pytest.mark.parametrize("kw", [dict(N=0), dict(N=10), dict(N=-1), dict(T=-1), dict(D_=0), dict(D_=7),
                                dict(D_=7172), dict(D_=ar.MAX_D + 8), dict(D_=-8), dict(eps=-1e-6),
                                dict(eps=float("nan")), dict(eps=float("inf")), dict(w=0), dict(src=0),
                                dict(out=0), dict(rstd=0), dict(alpha=0), dict(src=A + 8), dict(w=2 * A + 4),
                                dict(out=(1 << 36) + 2), dict(rstd=(1 << 36) + (1 << 30) + 2),
                                dict(T=1 << 40)],
                         ids=lambda k: ",".join(f"{a}={b}" for a, b in k.items()))
def test_fwd_rejects(kw):
    assert _fwd(**kw) == INVALID


def test_fwd_rejects_overlap():
    # out starting inside src
    assert _fwd(src=A, out=A + 16 * D) == INVALID
    # rstd overlapping alpha
    assert _fwd(rstd=1 << 38, alpha=(1 << 38) + 64) == INVALID
    # alpha overlapping w
    assert _fwd(alpha=2 * A) == INVALID


def test_fwd_T0_is_a_host_no_op():
    # nothing to do: returns before touching HIP; per-token pointers may be NULL
    assert _fwd(T=0, src=0, out=0, rstd=0, alpha=0) == OK
    # but w must still be valid
    assert _fwd(T=0, w=0) == INVALID


@pytest.mark.parametrize("kw", [dict(N=0), dict(N=10), dict(T=-5), dict(D_=12), dict(D_=ar.MAX_D + 8),
                                dict(dout=0), dict(src=0), dict(w=0), dict(rstd=0), dict(alpha=0), dict(dsrc=0),
                                dict(dw=0), dict(dout=(1 << 30) + 8), dict(dsrc=(8 << 30) + 4),
                                dict(dw=(12 << 30) + 4), dict(ws=(13 << 30) + 8), dict(rstd=(4 << 30) + 1)],
                         ids=lambda k: ",".join(f"{a}={b}" for a, b in k.items()))
def test_bwd_rejects(kw):
    assert _bwd(**kw) == INVALID


def test_bwd_workspace_errors():
    assert _bwd(ws=0) == WORKSPACE
    assert _bwd(ws_bytes=ar.workspace_bytes(16, 9, D) - 1) == WORKSPACE


def test_bwd_rejects_aliasing():
    g = 1 << 30
    assert _bwd(dsrc=2 * g) == INVALID  # dsrc == src
    assert _bwd(dsrc=g) == INVALID  # dsrc over dout
    assert _bwd(ws=2 * g + 64) == INVALID  # workspace inside src
    assert _bwd(dw=3 * g) == INVALID  # dw == w
    assert _bwd(dw=8 * g + 1024) == INVALID  # dw inside dsrc


def test_binding_refuses_host_tensors():
    import torch

    src = torch.zeros(2, 3, 8, dtype=torch.bfloat16)
    w = torch.zeros(8)
    with pytest.raises(ValueError):
        ar.attnres_fwd(src, w, 1e-6)


def test_binding_requires_one_device():
    """Every tensor of a call must sit on the sources' device (checked on the
    host, so testable without a GPU: meta/host tensors stand in)."""
    import torch

    dev = torch.device("cuda", 0)
    ar._same_device(dev, w=None)  # absent optional tensors are skipped
    with pytest.raises(ValueError, match="w is on cpu"):
        ar._same_device(dev, w=torch.zeros(8))
    with pytest.raises(ValueError, match=r"srcs\[1\]"):
        ar._same_device(torch.device("cpu"), **{"srcs[0]": torch.zeros(1), "srcs[1]": torch.zeros(1, device="meta")})


def _arr(vals):
    a = (ctypes.c_void_p * len(vals))()
    for i, v in enumerate(vals):
        a[i] = v
    return a


def _fwd_src(srcs, N=3, T=16, D_=D, eps=1e-6, w=2 * A, out=1 << 36, rstd=(1 << 36) + (1 << 30),
             alpha=(1 << 36) + (1 << 31), pitch=None):
    return ar.library().attnres_fwd_sources(srcs, D_ if pitch is None else pitch, w, eps, N, T, D_, out, rstd, alpha,
                                            None)


def test_fwd_sources_rejects():
    g = 1 << 30
    good = [g, 3 * g, 5 * g]
    assert _fwd_src(None) == INVALID
    assert _fwd_src(_arr([g, 0, 5 * g])) == INVALID  # null entry
    assert _fwd_src(_arr([g, 3 * g + 8, 5 * g])) == INVALID  # misaligned entry
    assert _fwd_src(_arr(good), out=3 * g + 64) == INVALID  # out inside a source
    assert _fwd_src(_arr(good), N=10) == INVALID
    assert _fwd_src(None, T=0) == OK  # nothing to do
    # the same source twice is a legal input (no output overlaps it)
    assert _fwd_src(_arr([g, g, 5 * g]), w=0) == INVALID  # still rejected, but only for the null w


def _bwd_src(srcs, dsrcs, acc=1, N=3, T=16, D_=D, ws_bytes=None, pitch=None, dpitch=None):
    g = 1 << 30
    if ws_bytes is None:
        ws_bytes = ar.workspace_bytes(T, max(N, 1), D_)
    return ar.library().attnres_bwd_sources(1 * g, srcs, D_ if pitch is None else pitch, 20 * g, 21 * g, 22 * g, N,
                                            T, D_, dsrcs, D_ if dpitch is None else dpitch, acc, 23 * g, 24 * g,
                                            ws_bytes, None)


def test_bwd_sources_rejects():
    g = 1 << 30
    srcs = _arr([2 * g, 3 * g, 4 * g])
    assert _bwd_src(srcs, None) == INVALID
    assert _bwd_src(None, _arr([8 * g, 9 * g, 10 * g])) == INVALID
    assert _bwd_src(srcs, _arr([8 * g, 8 * g, 10 * g])) == INVALID  # two gradients on one buffer
    assert _bwd_src(srcs, _arr([8 * g, 9 * g, 3 * g])) == INVALID  # gradient over a source
    assert _bwd_src(srcs, _arr([8 * g, 9 * g, g + 128])) == INVALID  # gradient over dout
    assert _bwd_src(srcs, _arr([8 * g, 9 * g + 2, 10 * g])) == INVALID  # misaligned
    assert _bwd_src(srcs, _arr([8 * g, 0, 10 * g])) == INVALID  # null entry
    assert _bwd_src(srcs, _arr([8 * g, 9 * g, 10 * g]), ws_bytes=8) == WORKSPACE


def _dec(srcs, N=3, T=16, D_=D, eps=1e-6, w=2 * A, out=1 << 36, rstd=(1 << 36) + (1 << 30),
         alpha=(1 << 36) + (1 << 31)):
    return ar.library().attnres_fwd_decode(srcs, D_, w, eps, N, T, D_, out, rstd, alpha, None)


def test_fwd_decode_rejects():
    g = 1 << 30
    good = _arr([g, 3 * g, 5 * g])
    assert _dec(None) == INVALID
    assert _dec(_arr([g, 0, 5 * g])) == INVALID  # null entry
    assert _dec(good, rstd=None) == INVALID  # saved state is both or neither
    assert _dec(good, alpha=None) == INVALID
    assert _dec(good, out=None, rstd=None, alpha=None) == INVALID  # out is always needed
    assert _dec(good, out=3 * g + 64) == INVALID  # out inside a source
    assert _dec(good, rstd=(1 << 36) + 8, alpha=(1 << 36) + 8 + 4 * 48) == INVALID  # rstd over out
    assert _dec(good, T=(1 << 31)) == INVALID  # one workgroup per token: T fits a 32-bit grid
    assert _dec(good, N=10) == INVALID
    assert _dec(good, D_=12) == INVALID
    assert _dec(good, w=0) == INVALID
    assert _dec(None, T=0) == OK  # nothing to do


def test_only_the_decode_call_may_skip_the_saved_state():
    g = 1 << 30
    assert _fwd(rstd=0, alpha=0) == INVALID
    assert _fwd_src(_arr([g, 3 * g, 5 * g]), rstd=None, alpha=None) == INVALID


def _upd(srcs, partial, delta, partial_out, N=3, T=16, D_=D, w=2 * A, out=1 << 36, rstd=(1 << 36) + (1 << 30),
         alpha=(1 << 36) + (1 << 31)):
    return ar.library().attnres_fwd_update(srcs, D_, partial, delta, w, 1e-6, N, T, D_, partial_out, out, rstd, alpha,
                                           None)


def test_fwd_update_rejects():
    g = 1 << 30
    srcs = _arr([g, 3 * g])
    p, y = 5 * g, 7 * g
    assert _upd(srcs, 0, y, p) == INVALID  # partial missing
    assert _upd(srcs, p, 0, p) == INVALID  # delta missing
    assert _upd(srcs, p, y, 0) == INVALID  # partial_out missing
    assert _upd(None, p, y, p) == INVALID  # N = 3 needs the two other sources
    assert _upd(srcs, p, y, p + 64) == INVALID  # partial_out overlapping partial, not equal to it
    assert _upd(srcs, p, y, y) == INVALID  # partial_out on delta
    assert _upd(srcs, p, y, 3 * g) == INVALID  # partial_out on another source
    assert _upd(_arr([g, p]), p, y, p) == INVALID  # in place while the partial sum is also another source
    assert _upd(srcs, p, y, 9 * g, out=9 * g + 128) == INVALID  # out overlapping partial_out
    assert _upd(srcs, p, y + 8, p) == INVALID  # misaligned delta
    assert _upd(srcs, p, y, p, rstd=None) == INVALID  # saved state is both or neither
    assert _upd(srcs, p, y, p, N=10) == INVALID
    assert _upd(None, p, y, p, T=0) == OK  # nothing to do


def test_source_pitch_rejects():
    g = 1 << 30
    good = _arr([g, 3 * g, 5 * g])
    assert _fwd_src(good, pitch=D - 8) == INVALID  # rows would overlap their successors
    assert _fwd_src(good, pitch=D + 4) == INVALID  # rows would lose 16-byte alignment
    assert _fwd_src(good, pitch=1 << 40) == INVALID  # offsets beyond the supported range
    # out inside the span of an interleaved source: spans are compared when pitches differ
    base = 7 * g
    inter = _arr([base, base + 2 * D, base + 4 * D])
    assert _fwd_src(inter, pitch=3 * D, out=base + 6 * D * 5) == INVALID


def test_interleaved_gradients_must_not_collide():
    g = 1 << 30
    srcs = _arr([2 * g, 3 * g, 4 * g])
    base = 8 * g
    # three gradients interleaved by token share a pitch of 3*D elements (6*D bytes)
    assert _bwd_src(srcs, _arr([base, base + D, base + 3 * D]), dpitch=3 * D) == INVALID  # 1st and 2nd overlap
    assert _bwd_src(srcs, _arr([base, base + 2 * D, base + 2 * D + 2 * D * 3 * 5]), dpitch=3 * D) == INVALID
    # gradients interleaved over a source cache that is interleaved the same way
    cache = 12 * g
    assert _bwd_src(_arr([cache, cache + 2 * D, cache + 4 * D]), _arr([cache + 2 * D, base, base + 2 * D]),
                    pitch=3 * D, dpitch=3 * D) == INVALID  # a gradient on a source row set


# ----------------------------------------------------------------------------
# argument-overlap validation against a byte-exact model (CPU only)
# ----------------------------------------------------------------------------
# A call whose arguments pass validation goes on to launch, which on a machine
# without a GPU fails with ATTNRES_ERR_HIP: that tells "accepted" (3) from
# "rejected" (1) without running anything.  The addresses are fake, so these
# tests must never run where a GPU is present.

def _no_gpu():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("passes fake device pointers to calls that would launch: CPU-only")


def _bytes(base, rows, row_bytes, pitch_bytes):
    return [(base + r * pitch_bytes, base + r * pitch_bytes + row_bytes) for r in range(rows)]


def _collide(a, b):
    return any(x0 < y1 and y0 < x1 for x0, x1 in a for y0, y1 in b)


def _span(a):
    return (a[0][0], a[-1][1])


def _layout(rng, n, T, Dv, arena):
    """n row sets of T rows of Dv bf16: either interleaved side by side (pitch
    n*Dv, phase offset chosen at random) or separate dense blocks at random
    16-byte positions of a small arena."""
    rb = 2 * Dv
    if rng.random() < 0.5:
        pitch = n * Dv
        base = arena + 16 * int(rng.integers(0, 64))
        slots = rng.permutation(n) if rng.random() < 0.7 else rng.integers(0, n, n)  # sometimes a shared slot
        return [base + int(k) * rb for k in slots], pitch
    pitch = int(rng.choice([Dv, 2 * Dv]))
    return [arena + 16 * int(rng.integers(0, 64)) for _ in range(n)], pitch


@pytest.mark.parametrize("seed", range(400))
def test_bwd_sources_overlap_checks_match_a_byte_model(seed):
    """Random small layouts of the sources, gradients and dout (interleaved or
    separate, in overlapping arenas): any pair of arguments sharing a byte that
    must not is rejected; any layout whose forbidden pairs have disjoint spans,
    or share one pitch and are byte-disjoint, is accepted."""
    _no_gpu()
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 4))
    T = int(rng.integers(1, 5))
    Dv = int(rng.choice([8, 16]))
    rb = Dv * 2
    arena = 1 << 32
    srcs, pitch = _layout(rng, N, T, Dv, arena)
    dsrcs, dpitch = _layout(rng, N, T, Dv, arena + 16 * int(rng.integers(0, 64)))
    dout = arena + 16 * int(rng.integers(0, 256)) if rng.random() < 0.3 else (1 << 33)
    wsb = ar.workspace_bytes(T, N, Dv)
    dw = arena + 16 * int(rng.integers(0, 256)) if rng.random() < 0.2 else (1 << 33) + (1 << 24)
    ws = arena + 16 * int(rng.integers(0, 256)) if rng.random() < 0.2 else (1 << 33) + (1 << 25)
    w, rstd, alpha = (1 << 34), (1 << 35), (1 << 35) + (1 << 20)
    ins = [_bytes(s, T, rb, 2 * pitch) for s in srcs] + [_bytes(dout, T, rb, rb), _bytes(w, 1, 4 * Dv, 4 * Dv)]
    outs = [_bytes(d, T, rb, 2 * dpitch) for d in dsrcs] + [_bytes(dw, 1, 4 * Dv, 4 * Dv), _bytes(ws, 1, wsb, wsb)]
    pitches_in = [2 * pitch] * N + [None, None]
    pitches_out = [2 * dpitch] * N + [None, None]
    pairs = [(o, i, po, pi) for o, po in zip(outs, pitches_out) for i, pi in zip(ins, pitches_in)]
    pairs += [(outs[a], outs[b], pitches_out[a], pitches_out[b])
              for a in range(len(outs)) for b in range(a + 1, len(outs))]
    collide = any(_collide(a, b) for a, b, _, _ in pairs)

    def clearly_ok(a, b, pa, pb):
        (a0, a1), (b0, b1) = _span(a), _span(b)
        if not (a0 < b1 and b0 < a1):
            return True
        return pa is not None and pa == pb and len(a) > 1 and len(b) > 1 and not _collide(a, b)

    must_accept = all(clearly_ok(*p) for p in pairs)
    code = ar.library().attnres_bwd_sources(dout, _arr(srcs), pitch, w, rstd, alpha, N, T, Dv, _arr(dsrcs), dpitch,
                                            0, dw, ws, wsb, None)
    assert code in (INVALID, 3)
    if collide:
        assert code == INVALID, "an overlapping layout was accepted"
    elif must_accept:
        assert code == 3, "a disjoint layout was rejected"


def test_bwd_sources_rejects_unknown_grad_modes():
    g = 1 << 30
    srcs, dsrcs = _arr([2 * g, 3 * g, 4 * g]), _arr([8 * g, 9 * g, 10 * g])
    assert _bwd_src(srcs, dsrcs, acc=4) == INVALID
    assert _bwd_src(srcs, dsrcs, acc=-1) == INVALID
    assert _bwd_src(srcs, dsrcs, acc=7, T=0) == INVALID  # checked before the empty-batch shortcut


def test_grad_mode_constants_match_binding():
    assert _define("ATTNRES_GRAD_BF16") == 0
    assert _define("ATTNRES_GRAD_ACCUMULATE") == ar.GRAD_ACCUMULATE
    assert _define("ATTNRES_GRAD_F32") == ar.GRAD_F32


PROBE_HEADER = os.path.join(ROOT, "include", "attnres_probes.h")
PROBE_LIB = os.path.join(ROOT, "attention_residuals_depth_amd", "libattnres_probes.so")


def test_probe_library_exports_declared_symbols_and_refuses_bad_arguments():
    names = re.findall(r"^int\s+(attnres_probe_\w+)\s*\(", open(PROBE_HEADER).read(), re.M)
    assert names == ["attnres_probe_read", "attnres_probe_write", "attnres_probe_copy", "attnres_probe_fwd_pattern",
                     "attnres_probe_bwd_pattern", "attnres_probe_split_bwd_pattern"]
    lib = ctypes.CDLL(PROBE_LIB)
    out = subprocess.run(["nm", "-D", "--defined-only", PROBE_LIB], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported
    vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    lib.attnres_probe_read.argtypes = [vp, sz, vp, vp]
    lib.attnres_probe_copy.argtypes = [vp, vp, sz, vp]
    lib.attnres_probe_fwd_pattern.argtypes = [vp, i32, i64, i32, vp, vp]
    # invalid arguments are refused on the host (status 1), nothing is enqueued
    assert lib.attnres_probe_read(None, 4096, A, None) == 1
    assert lib.attnres_probe_read(A + 8, 4096, A, None) == 1      # misaligned
    assert lib.attnres_probe_read(A, 4100, A, None) == 1          # not a multiple of 16
    assert lib.attnres_probe_copy(A, A + 4096, 8192, None) == 1   # overlapping
    ptrs = (ctypes.c_void_p * 9)(*([A] * 9))
    assert lib.attnres_probe_fwd_pattern(ptrs, 10, 16, D, A, None) == 1   # N > 9
    assert lib.attnres_probe_fwd_pattern(ptrs, 9, 16, 8200, A, None) == 1  # D > 8192
    lib.attnres_probe_split_bwd_pattern.argtypes = [vp, vp, i32, i64, i32, vp, vp, vp]
    assert lib.attnres_probe_split_bwd_pattern(ptrs, A, 9, 16, D, ptrs, None, None) == 1      # no partial rows
    assert lib.attnres_probe_split_bwd_pattern(ptrs, A, 9, 16, D, ptrs, A + 4, None) == 1     # misaligned
    assert lib.attnres_probe_read(A, 0, A, None) == 0              # empty: nothing to do


def test_noalloc_backward_refuses_on_the_host():
    """attnres_bwd_noalloc: the static partial rows hold D <= 8192, a larger D is
    ATTNRES_ERR_WORKSPACE; the shared argument checks of attnres_bwd apply
    first.  Nothing reaches the GPU (every call has an invalid argument)."""
    lib = ar.library()
    g = 1 << 30

    def call(N=9, T=16, D_=D, dw=12 * g, w=3 * g, src=2 * g):
        return lib.attnres_bwd_noalloc(1 * g, src, w, 4 * g, 5 * g, N, T, D_, 8 * g, dw, None)

    assert call(D_=8200) == WORKSPACE
    assert call(D_=16384) == WORKSPACE
    assert call(N=10) == INVALID
    assert call(D_=7170) == INVALID
    assert call(dw=0) == INVALID
    assert call(w=12 * g) == INVALID  # dw overlaps w
    assert call(T=-1) == INVALID


def test_split_spin_setter_returns_the_previous_bound():
    """attnres_set_split_spin is host state only (no GPU): it swaps the bound."""
    assert ar.set_split_spin(7) == ar.SPLIT_SPIN_DEFAULT
    assert ar.set_split_spin(0) == 7
    assert ar.set_split_spin(ar.SPLIT_SPIN_DEFAULT) == 0
    with pytest.raises(ValueError):
        ar.set_split_spin(-1)


def test_workspace_macro_matches_binding(tmp_path):
    """ATTNRES_BWD_WORKSPACE_BYTES, compiled by a plain C compiler, gives the
    binding's workspace_bytes at the chunk and split boundaries."""
    cases = [(T, N, D_) for T in (0, 1, 3, 4, 5, 32763, 32764, 32765, 32768, 32769, 131072, 262147)
             for N in (1, 7, 8, 9) for D_ in (8, 1024, 1032, 7168, 7176, 8192, 8200, 16384)]
    src = tmp_path / "ws.c"
    body = "\n".join(f'  printf("%zu\\n", (size_t)ATTNRES_BWD_WORKSPACE_BYTES({T}LL, {N}, {D_}));' for T, N, D_ in cases)
    src.write_text(f'#include <stdio.h>\n#include "attnres.h"\nint main(void) {{\n{body}\n  return 0;\n}}\n')
    exe = tmp_path / "ws"
    inc = os.path.join(ROOT, "include")
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", inc,
                    "-o", str(exe), str(src)], check=True, capture_output=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    assert got == [ar.workspace_bytes(T, N, D_) for T, N, D_ in cases]


def test_decode_u24_reads_the_24_bit_format():
    """decode_u24 (host logic, CPU tensors here) reads the 24-bit elements as
    the oracle's decode24 does, on every byte pattern of a random sample and
    on the oracle's encodings of random values (within 2^-16 relative of the
    values, infinity where they round past the binary32 range)."""
    import torch
    import oracle
    rng = np.random.default_rng(3)
    raw = rng.integers(0, 256, (5000, 3)).astype(np.uint8)
    assert np.array_equal(ar.decode_u24(torch.from_numpy(raw)).numpy().view(np.uint32),
                          oracle.decode24(raw).view(np.uint32))
    v = (rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000)).astype(np.float32)
    enc = oracle.round24(v)
    d = ar.decode_u24(torch.from_numpy(enc)).numpy()
    assert np.array_equal(d.view(np.uint32), oracle.decode24(enc).view(np.uint32))
    assert np.all(np.abs(d.astype(np.float64) - v) <= 2.0 ** -16 * np.abs(v.astype(np.float64)))
    with pytest.raises(ValueError):
        ar.decode_u24(torch.zeros((4, 2), dtype=torch.uint8))

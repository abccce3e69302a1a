"""The ABI from plain C: tests/c/abi_check (built by __graft_entry__.build())
allocates with hipMalloc, calls attnres_fwd / attnres_bwd / attnres_fwd_sources
directly and checks the results against the fp64 oracle; it runs here as a
child process."""
from __future__ import annotations

import os
import subprocess

import pytest
import torch

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "abi_check")


def test_c_consumer_of_the_abi():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(BIN):
        raise RuntimeError(f"{BIN} is missing: build it with __graft_entry__.build()")
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr

"""The library driven from plain C: tests/c_abi/decode_from_c.c (built by
build() with gcc as C99 against the in-tree libdf11.so, through
include/df11.h and the HIP runtime API only) encodes three seeded tensors on
the host, plans and decodes them in one batched launch on a stream of its
own, checks the flag, compares every word with its source, and compares the
GPU encoder's containers with the host encoder's."""
import os
import subprocess

import pytest

from gpu_util import log

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "decode_from_c")


def test_decode_from_a_c_program():
    assert os.path.exists(BIN), "tests/c_abi/decode_from_c is not built: run __graft_entry__.build()"
    log("C program over the C ABI")
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("ok: 3 tensors")

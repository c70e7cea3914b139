"""Properties of the compiled gfx950 decode kernel that its speed depends on
and that a small source change can lose without any test failing:

  * no scratch: a kernel that spills even a few bytes per lane gets private
    memory set up for every wave;
  * no flat memory instructions: a flat store also counts against the LDS
    wait counter, so each LDS wait after it waits for the store to reach
    memory (the assembly of a chunk then runs one store at a time);
  * three waves per SIMD: three workgroups per compute unit, as the LDS
    layout is sized for.

The kernel is compiled to assembly here with the same flags as the build."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lossless_bf16_weight_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _compile(src, tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path / "k.s"
    r = subprocess.run([HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature",
                        "-Xclang", "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
                        "--cuda-device-only", "-S", "-o", str(out), os.path.join(CSRC, src),
                        "-Rpass-analysis=kernel-resource-usage"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text(), r.stderr


def _remark(stderr, name):
    m = re.findall(name + r" \[[^]]*\]: (\d+)|" + name + r": (\d+)", stderr)
    assert m, name
    return [int(a or b) for a, b in m]


@pytest.mark.parametrize("src", ["decode.hip", "nf12.hip", "control.hip", "encode_gpu.hip"])
def test_no_scratch_and_no_flat_memory(src, tmp_path):
    asm, remarks = _compile(src, tmp_path)
    assert all(v == 0 for v in _remark(remarks, r"ScratchSize \[bytes/lane\]")), src
    flat = re.findall(r"^\s*flat_(load|store|atomic)\w*", asm, re.M)
    assert not flat, (src, flat[:5])


def test_decode_kernel_three_waves_per_simd(tmp_path):
    _, remarks = _compile("decode.hip", tmp_path)
    assert _remark(remarks, r"Occupancy \[waves/SIMD\]") == [3]

"""The documented build entry point, run end to end on the CPU: it compiles
libdf11.so for gfx950, the C program over the C ABI and the oracles with
gcc, loads the library and checks that its ABI version is the one the
Python binding marshals for."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_graft_entry_build_runs_end_to_end():
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    r = subprocess.run([sys.executable, "-c", "import __graft_entry__ as g; g.build()"], cwd=ROOT,
                       capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    import lossless_bf16_weight_amd as df11
    assert df11.lib().df11_abi_version() == df11.ABI_VERSION
    # and the C program over the C ABI (run by the GPU tests)
    example = os.path.join(ROOT, "tests", "c_abi", "decode_from_c")
    assert os.path.exists(example) and os.access(example, os.X_OK)


def test_binding_abi_version_matches_header():
    import re
    text = open(os.path.join(ROOT, "include", "df11.h")).read()
    m = re.search(r"#define\s+DF11_ABI_VERSION\s+(\d+)", text)
    import lossless_bf16_weight_amd as df11
    assert m and int(m.group(1)) == df11.ABI_VERSION

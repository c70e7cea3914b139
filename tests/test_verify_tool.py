"""The verify tool's levels and exit codes (df11pack project page, "Use":
structure with no source, sampled chunks decoded against the source, or
everything at the full level; exit 0 pass, 1 a check failed, 2 could not
check).  The structure level and every "could not check" case run on the
CPU; the decoding levels run on the GPU."""
import os
import subprocess
import sys

import numpy as np
import pytest

import lossless_bf16_weight_amd as df11
from lossless_bf16_weight_amd import verify_tool as V
from lossless_bf16_weight_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _files(tmp_path, words_list, sha=False):
    paths, srcs = [], []
    for k, w in enumerate(words_list):
        c = df11.encode(w, sha256=sha)
        p = tmp_path / f"t{k}.df11"
        c.tofile(p)
        s = tmp_path / f"t{k}.npy"
        np.save(s, w)
        paths.append(str(p))
        srcs.append(str(s))
    return paths, srcs


def _tensors():
    return [W.normal_bf16((3 * 32768 + 123,), seed=3), W.normal_bf16((70000,), seed=4)]


def test_structure_level_passes(tmp_path):
    paths, _ = _files(tmp_path, _tensors())
    assert V.main(paths) == V.PASS


def test_structure_level_fails_on_a_broken_index(tmp_path):
    paths, _ = _files(tmp_path, _tensors())
    c = np.fromfile(paths[1], np.uint8)
    info = df11.validate(c)
    # one window entry of chunk 0 made to count one code more than it holds
    off_win = int(c[120:128].view(np.uint64)[0])
    e = int(c[off_win + 2 * 7:off_win + 2 * 8].view(np.uint16)[0])
    c[off_win + 2 * 7:off_win + 2 * 8] = np.array([e + 1], np.uint16).view(np.uint8)
    assert info["n_chunks"] >= 1
    c.tofile(paths[1])
    assert V.main(paths) == V.FAIL


def test_structure_level_fails_on_a_truncated_container(tmp_path):
    paths, _ = _files(tmp_path, _tensors())
    c = np.fromfile(paths[0], np.uint8)
    c[: c.size - 4096].tofile(paths[0])
    assert V.main(paths) == V.FAIL


def test_could_not_check(tmp_path):
    paths, srcs = _files(tmp_path, _tensors())
    # a file that is not there
    assert V.main([str(tmp_path / "missing.df11")]) == V.CANNOT
    # a container version this build does not decode
    c = np.fromfile(paths[0], np.uint8)
    c[8:12] = np.array([3], np.uint32).view(np.uint8)
    c.tofile(tmp_path / "v3.df11")
    assert V.main([str(tmp_path / "v3.df11")]) == V.CANNOT
    # sampled chunks need a source
    assert V.main(paths + ["--level", "sampled"]) == V.CANNOT
    # the full level needs a source or a hash in every header
    assert V.main(paths + ["--level", "full"]) == V.CANNOT
    # one source for two containers
    assert V.main(paths + ["--source", srcs[0]]) == V.CANNOT


def test_could_not_check_without_a_gpu(tmp_path):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    paths, srcs = _files(tmp_path, _tensors())
    assert V.main(paths + ["--source"] + srcs) == V.CANNOT


def test_command_line_exit_codes(tmp_path):
    paths, _ = _files(tmp_path, _tensors())
    r = subprocess.run([sys.executable, "-m", "lossless_bf16_weight_amd.verify_tool"] + paths, cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "PASS" in r.stdout
    r = subprocess.run([sys.executable, "-m", "lossless_bf16_weight_amd.verify_tool", str(tmp_path / "none")],
                       cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2


@pytest.mark.gpu
def test_sampled_level_on_the_gpu(tmp_path):
    ws = _tensors()
    paths, srcs = _files(tmp_path, ws)
    assert V.main(paths + ["--source"] + srcs) == V.PASS
    # a source word changed: every chunk sampled, so the differing one is seen
    w = ws[1].copy()
    w[40000] ^= 0x0001
    np.save(srcs[1], w)
    assert V.main(paths + ["--source"] + srcs + ["--samples", "100000"]) == V.FAIL


@pytest.mark.gpu
def test_full_level_on_the_gpu(tmp_path):
    ws = _tensors()
    paths, srcs = _files(tmp_path, ws, sha=True)
    assert V.main(paths + ["--level", "full"]) == V.PASS
    assert V.main(paths + ["--level", "full", "--source"] + srcs) == V.PASS
    # one fraction bit flipped in the raw section: the structure still
    # passes, the decoded words differ from the source and from the hash
    c = np.fromfile(paths[0], np.uint8)
    off_raw = int(c[152:160].view(np.uint64)[0])
    c[off_raw + 5] ^= 0x01
    c.tofile(paths[0])
    assert V.main(paths) == V.PASS
    assert V.main(paths + ["--level", "full"]) == V.FAIL
    assert V.main(paths + ["--level", "full", "--source"] + srcs) == V.FAIL

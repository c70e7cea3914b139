"""Build libdf11.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdf11.so")
BUILD = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I" + os.path.join(ROOT, "include")]
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

SOURCES = [
    ("host.cpp", ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"]),
    ("encode.cpp", ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"]),
    ("sha256.cpp", ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"]),
    ("decode.hip", DEVICE),
    ("control.hip", DEVICE),
    ("nf12.cpp", ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"]),
    ("nf12.hip", DEVICE),
    ("encode_gpu.hip", DEVICE),
]


def _compile(item):
    src, extra = item
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC] + COMMON + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


C_EXAMPLE = os.path.join(ROOT, "tests", "c_abi", "decode_from_c.c")


def build_c_example() -> str:
    """The C program that drives the library through include/df11.h alone
    (tests/c_abi), built with gcc as C99 against the in-tree libdf11.so."""
    out = C_EXAMPLE[:-2]
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), C_EXAMPLE, "-L" + PKG, "-ldf11",
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../lossless_bf16_weight_amd",
           "-Wl,-rpath,/opt/rocm/lib", "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C example build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs + ["-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    example = build_c_example()
    if verbose:
        print("built", LIB)
        print("built", example)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

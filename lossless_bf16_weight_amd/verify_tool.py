"""Check DF11 containers, with the df11pack page's three levels and exit codes.

The df11pack project page ("Use") describes a verify command that checks the
structure of compressed files with no source at hand, adds a decode of 1000
sampled chunks compared with the source when the source is given, or decodes
everything at `--level full`; it exits 0 when every check passes, 1 when a
check fails and 2 when it could not check.  The same here, for containers of
this library:

  structure  df11_validate over every whole container (header, code lengths
             and Kraft sum, chunk and window index, stream padding); no GPU
  sampled    structure, then a GPU decode of the containers; `--samples`
             chunks drawn (seeded) over all tensors are compared word for word
             with the source; the decode's corruption flag must stay clear
  full       structure, then every decoded word is compared with the source
             and, for a container whose header holds the source's SHA-256
             (df11pack page, "Beyond the official format", per-tensor
             hashes), checked against that hash; with neither a source nor a
             hash a tensor cannot be checked past its structure

Containers are files of container bytes; sources are .npy files (or raw
little-endian files) of the tensors' 16-bit words, one per container, in the
same order.  Every decode runs in libdf11 on the GPU: this module only reads
files, calls the library and compares words.

    python -m lossless_bf16_weight_amd.verify_tool a.df11 b.df11 --source a.npy b.npy
"""
from __future__ import annotations

import argparse
import os
import sys
from typing import List, Optional, Sequence, Tuple

import numpy as np

PASS, FAIL, CANNOT = 0, 1, 2


def _read_container(path: str) -> np.ndarray:
    return np.fromfile(path, dtype=np.uint8)


def _read_source(path: str) -> np.ndarray:
    """A source tensor's 16-bit words (memory-mapped, nothing is unpickled)."""
    if path.endswith(".npy"):
        a = np.load(path, mmap_mode="r", allow_pickle=False)
        if a.dtype.itemsize != 2:
            raise ValueError(f"{path}: {a.dtype} is not a 16-bit dtype")
        return a.reshape(-1).view(np.uint16)
    return np.memmap(path, dtype=np.uint16, mode="r")


def _has_hash(info: dict) -> bool:
    from ._lib import FLAG_SHA256
    return bool(info["flags"] & FLAG_SHA256)


def verify_containers(containers: Sequence[np.ndarray], sources: Optional[Sequence[np.ndarray]] = None,
                      level: str = "structure", samples: int = 1000, seed: int = 0,
                      device: int = 0, names: Optional[Sequence[str]] = None) -> Tuple[int, List[str]]:
    """Check host copies of whole containers; returns (exit code, messages)."""
    from . import _lib as L

    names = list(names) if names is not None else [f"tensor {i}" for i in range(len(containers))]
    msgs: List[str] = []
    if level not in ("structure", "sampled", "full"):
        return CANNOT, [f"unknown level {level!r}"]
    if sources is not None and len(sources) != len(containers):
        return CANNOT, [f"{len(sources)} sources for {len(containers)} containers"]

    # ---- structure (no source, no GPU)
    infos = []
    worst = PASS
    for name, c in zip(names, containers):
        st = L.validate_status(c)
        if st == L.OK:
            info = L.validate(c)
            if c.size == info["container_bytes"]:
                infos.append(info)
                continue
            msgs.append(f"{name}: {c.size} bytes, the header gives {info['container_bytes']}")
            worst = max(worst, FAIL)
            infos.append(None)
            continue
        text = L.lib().df11_last_error().decode()
        if st in (L.E_FORMAT,):
            msgs.append(f"{name}: structure check failed: {text}")
            worst = max(worst, FAIL)
        else:
            msgs.append(f"{name}: could not check the structure ({L.lib().df11_status_str(st).decode()}): {text}")
            worst = max(worst, CANNOT)
        infos.append(None)
    if worst != PASS or level == "structure":
        if worst == PASS:
            msgs.append(f"structure: {len(containers)} container(s) pass")
        return worst, msgs

    if sources is not None:
        for name, info, s in zip(names, infos, sources):
            if s.size != info["n_elems"]:
                msgs.append(f"{name}: the source holds {s.size} words, the container {info['n_elems']}")
                return FAIL, msgs
    if level == "sampled" and sources is None:
        return CANNOT, msgs + ["sampled level: no source to compare the sampled chunks with"]
    if level == "full" and sources is None and not all(_has_hash(i) for i in infos):
        return CANNOT, msgs + ["full level: no source, and not every header holds the source's SHA-256"]

    # ---- decode on the GPU
    try:
        import torch
        if not torch.cuda.is_available():
            return CANNOT, msgs + [f"{level} level: no GPU to decode on"]
    except ImportError:
        return CANNOT, msgs + [f"{level} level: torch is not available"]
    dev = torch.device("cuda", device)
    plan = L.Plan(list(containers), device=device)
    try:
        d_conts = [torch.from_numpy(np.ascontiguousarray(c)).to(dev) for c in containers]
        outs = [torch.empty(i["n_elems"], dtype=torch.int16, device=dev) for i in infos]
        stream = torch.cuda.current_stream(dev)
        L.decode_batch(plan, d_conts, outs, stream=stream)
        try:
            L.check(plan, stream=stream)
        except L.DF11Error as e:
            msgs.append(f"decode: {e}")
            worst = FAIL

        if level == "sampled":
            chunks = [(t, c) for t, i in enumerate(infos) for c in range(i["n_chunks"])]
            rng = np.random.default_rng(seed)
            pick = chunks if samples >= len(chunks) else [chunks[k] for k in
                                                          sorted(rng.choice(len(chunks), samples, replace=False))]
            bad = 0
            for t, c in pick:
                lo, hi = c * 32768, min((c + 1) * 32768, infos[t]["n_elems"])
                want = torch.from_numpy(np.array(sources[t][lo:hi], dtype=np.uint16).view(np.int16)).to(dev)
                if not torch.equal(outs[t][lo:hi], want):
                    bad += 1
                    if bad <= 5:
                        msgs.append(f"{names[t]}: chunk {c} decodes to words that differ from the source")
            msgs.append(f"sampled: {len(pick)} chunk(s) compared, {bad} differ")
            if bad:
                worst = FAIL
        else:
            for t, info in enumerate(infos):
                got = outs[t].cpu().numpy().view(np.uint16)
                if sources is not None:
                    diff = int(np.count_nonzero(got != np.asarray(sources[t])))
                    if diff:
                        msgs.append(f"{names[t]}: {diff} decoded word(s) differ from the source")
                        worst = FAIL
                if _has_hash(info):
                    st = L.verify_status(containers[t], got)
                    if st == L.E_CORRUPT:
                        msgs.append(f"{names[t]}: the decoded words' SHA-256 differs from the header's")
                        worst = FAIL
                    elif st != L.OK:
                        msgs.append(f"{names[t]}: could not check the hash ({L.lib().df11_status_str(st).decode()})")
                        worst = max(worst, CANNOT)
            msgs.append(f"full: {len(infos)} tensor(s) decoded and compared")
    finally:
        plan.close()
    return worst, msgs


def main(argv: Optional[Sequence[str]] = None) -> int:
    ap = argparse.ArgumentParser(prog="python -m lossless_bf16_weight_amd.verify_tool",
                                 description="Check DF11 containers (exit 0 pass, 1 a check failed, "
                                             "2 could not check).")
    ap.add_argument("containers", nargs="+")
    ap.add_argument("--source", nargs="+", default=None,
                    help="the source tensors (.npy or raw 16-bit words), one per container")
    ap.add_argument("--level", choices=("structure", "sampled", "full"), default=None,
                    help="default: sampled with --source, else structure")
    ap.add_argument("--samples", type=int, default=1000)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--device", type=int, default=0)
    args = ap.parse_args(argv)
    level = args.level or ("sampled" if args.source else "structure")
    try:
        conts = [_read_container(p) for p in args.containers]
        srcs = [_read_source(p) for p in args.source] if args.source else None
    except (OSError, ValueError) as e:
        print(f"verify: could not read the input: {e}", file=sys.stderr)
        return CANNOT
    try:
        code, msgs = verify_containers(conts, srcs, level=level, samples=args.samples, seed=args.seed,
                                       device=args.device, names=[os.path.basename(p) for p in args.containers])
    except ImportError as e:   # the library is not built
        print(f"verify: could not check: {e}", file=sys.stderr)
        return CANNOT
    for m in msgs:
        print(m)
    print({PASS: "PASS", FAIL: "FAIL", CANNOT: "COULD NOT CHECK"}[code])
    return code


if __name__ == "__main__":
    sys.exit(main())

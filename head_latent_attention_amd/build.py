"""Compile the gfx950 MLA library (libmla.so) in-tree with hipcc.

Every ``csrc/*.hip`` file is compiled for gfx950 only, then linked into
``head_latent_attention_amd/libmla.so``; the measurement probes of ``peaks/`` (streaming
read/copy and a matrix-op loop, used by the benchmark only) go into ``libmla_peaks.so``.
Run as ``python -m head_latent_attention_amd.build`` or call :func:`build`.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmla.so")
PEAKS_SRC = os.path.join(PKG, "peaks")
PEAKS_LIB = os.path.join(PKG, "libmla_peaks.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Wno-unused-variable", "-Wno-unused-but-set-variable",
    # packed fp32 VALU instructions are kept off for every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def sources(folder: str = CSRC):
    return sorted(os.path.join(folder, f) for f in os.listdir(folder) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(os.path.dirname(src)) + "_" + os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed for {lib}:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    """Compile every source and link libmla.so and libmla_peaks.so; returns libmla.so's path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs, psrcs = sources(), sources(PEAKS_SRC)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(psrcs))) as ex:
        objs = list(ex.map(_compile, srcs + psrcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PEAKS_LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources and {PEAKS_LIB} from {len(psrcs)}")
    return LIB


if __name__ == "__main__":
    build()

"""Build libtattn.so (the HIP kernels + C ABI) in-tree with hipcc for gfx950.

Usage: ``python -m tiled_attention_10_amd.build`` (or ``build()`` from Python).
Objects go to ``_build/`` at the repository root; the library is written next
to this file so that it travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtattn.so")

ARCH = "gfx950"
# Packed fp32 VALU forms are kept out of the generated code on purpose.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-function"]
SOURCES = ["attn_fwd16.hip", "attn_fwd_fp8.hip", "attn_decode.hip", "hadamard.hip", "api.cpp"]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [_hipcc(), *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


PROBE_SRC = os.path.join(CSRC, "measure", "clock_probe.hip")
PROBE_LIB = os.path.join(PKG, "libtattn_clock.so")


def build_probe(verbose: bool = False) -> str:
    """The benchmark's shader-clock probe, a library of its own (not part of the ABI)."""
    cmd = [_hipcc(), *FLAGS, "-shared", PROBE_SRC, "-o", PROBE_LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for the clock probe:\n{r.stderr}")
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return PROBE_LIB


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library (and the benchmark's clock
    probe); returns the library's path."""
    os.makedirs(OBJDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    build_probe(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

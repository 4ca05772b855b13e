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

# Scheduling variants of the 16-bit kernel for the ablation: each is the whole
# library with attn_fwd16.hip rebuilt under other schedule settings, written to
# libtattn_<name>.so.  The shipped library uses the defaults in attn_fwd16.hip
# (4-stage rings, reads 2 products ahead, two-group ping-pong, split loads,
# scale applied in fp32).
VARIANTS = {
    "stages3": ["-DTATTN_STAGES=3"],
    "stages5": ["-DTATTN_STAGES=5"],
    "uniform": ["-DTATTN_PINGPONG=0"],
    "readahead1": ["-DTATTN_READ_AHEAD=1"],
    "readahead4": ["-DTATTN_READ_AHEAD=4"],
    "loads_at_barrier": ["-DTATTN_SPLIT_LOADS=0"],
    "foldscale": ["-DTATTN_FOLD_SCALE=1"],
}
# Variants whose arithmetic differs from the shipped build (not bit-identical to it).
ARITH_VARIANTS = {"foldscale"}
# Variants of the fp8 kernel (attn_fwd_fp8.hip rebuilt, libtattn_<name>.so): part of
# every 8 exponentials of a full tile on the VALU pipe (exp2_valu) instead of
# v_exp_f32, or the LDS operand reads issued 3 or 4 products ahead instead of 2.
# The shipped library computes every exponential with v_exp_f32 and reads 2 ahead.
FP8_VARIANTS = {
    "fp8_expvalu1": ["-DTATTN_FP8_EXP_VALU=1"],
    "fp8_expvalu2": ["-DTATTN_FP8_EXP_VALU=2"],
    "fp8_expvalu4": ["-DTATTN_FP8_EXP_VALU=4"],
    "fp8_readahead3": ["-DTATTN_FP8_READ_AHEAD=3"],
    "fp8_readahead4": ["-DTATTN_FP8_READ_AHEAD=4"],
}


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src: str, verbose: bool, variant: str | None = None) -> str:
    stem = os.path.splitext(src)[0] + ("" if variant is None else "_" + variant)
    obj = os.path.join(OBJDIR, stem + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    extra = [] if variant is None else {**VARIANTS, **FP8_VARIANTS}[variant]
    cmd = [_hipcc(), *FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
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


def variant_lib(name: str) -> str:
    return os.path.join(PKG, f"libtattn_{name}.so")


def _link(objs, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, variants: bool = True) -> str:
    """Compile every source and link the shared library, the scheduling variants
    (unless ``variants`` is False) and the benchmark's clock probe; returns the
    library's path."""
    os.makedirs(OBJDIR, exist_ok=True)
    var_jobs = ([("attn_fwd16.hip", v) for v in VARIANTS] + [("attn_fwd_fp8.hip", v) for v in FP8_VARIANTS]
                if variants else [])
    jobs = [(s, None) for s in SOURCES] + var_jobs
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1]), jobs))
    base = objs[:len(SOURCES)]
    _link(base, LIB, verbose)
    for (src, v), obj in zip(var_jobs, objs[len(SOURCES):]):
        i = SOURCES.index(src)
        _link(base[:i] + [obj] + base[i + 1:], variant_lib(v), verbose)
    build_probe(verbose)
    return LIB


def resource_usage(verbose: bool = False, sources=None) -> str:
    """Per-kernel register, scratch, occupancy and LDS use of the given sources (default
    all) and the variants of attn_fwd16.hip and attn_fwd_fp8.hip among them, from the
    compiler's kernel-resource-usage remarks (a markdown table)."""
    import re
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = [s for s in SOURCES if s.endswith(".hip") and (not sources or s in sources)]
    jobs = ([(s, None) for s in srcs] + ([("attn_fwd16.hip", v) for v in VARIANTS] if "attn_fwd16.hip" in srcs else [])
            + ([("attn_fwd_fp8.hip", v) for v in FP8_VARIANTS] if "attn_fwd_fp8.hip" in srcs else []))

    def one(job):
        src, var = job
        extra = [] if var is None else {**VARIANTS, **FP8_VARIANTS}[var]
        cmd = [_hipcc(), *FLAGS, *extra, "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src),
               "-o", os.path.join(OBJDIR, "resource_usage_tmp_" + (var or "") + os.path.splitext(src)[0] + ".o")]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        rows, cur = [], None
        for line in r.stderr.splitlines():
            m = re.search(r"remark:\s+(Function Name|VGPRs|AGPRs|TotalSGPRs|ScratchSize \[bytes/lane\]|"
                          r"Occupancy \[waves/SIMD\]|LDS Size \[bytes/block\]): (\S+)", line)
            if not m:
                continue
            key, val = m.group(1).split(" [")[0], m.group(2)
            if key == "Function Name":
                cur = {"kernel": val}
                rows.append(cur)
            elif cur is not None:
                cur[key] = val
        return src, var, rows

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        results = list(ex.map(one, jobs))
    out = ["| source | variant | kernel | VGPRs | AGPRs | SGPRs | scratch B/lane | waves/SIMD | LDS B |",
           "|---|---|---|---|---|---|---|---|---|"]
    for src, var, rows in results:
        for r in rows:
            out.append(f"| {src} | {var or 'shipped'} | `{r['kernel']}` | {r.get('VGPRs')} | {r.get('AGPRs')} | "
                       f"{r.get('TotalSGPRs')} | {r.get('ScratchSize')} | {r.get('Occupancy')} | {r.get('LDS Size')} |")
    return "\n".join(out)


if __name__ == "__main__":
    if "--resource-usage" in sys.argv:
        print(resource_usage(verbose="-v" in sys.argv, sources=[a for a in sys.argv[1:] if a.endswith(".hip")]))
        sys.exit(0)
    print(build(verbose="-v" in sys.argv, variants="--no-variants" not in sys.argv))

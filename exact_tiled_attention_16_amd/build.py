"""Build libfa.so in-tree with hipcc for gfx950.

``python -m exact_tiled_attention_16_amd.build`` (or ``build()``) compiles
every translation unit under ``csrc/`` to an object in ``_build/`` at the
repository root and links ``exact_tiled_attention_16_amd/libfa.so`` (and the
clock probe used by bench.py, ``libfa_probe.so``, and the instruction-rate
probe program ``isa_probe``, a measurement aid).  It always
recompiles; loading code never builds.  The device assembly of the sources
with LDS-DMA copies is checked for the copies' wait states (asmcheck.py);
a copy without them fails the build.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
# Measurement aid used by bench.py (shader clock under load); not part of the
# attention library.
PROBE_SOURCE = "clock_probe.hip"
PROBE_LIB = os.path.join(PKG, "libfa_probe.so")
# Measurement aid: a standalone program timing the instructions the kernels
# are built from (isa_probe.hip); not part of the library.
RATE_SOURCE = "isa_probe.hip"
RATE_EXE = os.path.join(PKG, "isa_probe")

ARCH = "gfx950"
SOURCES = ["fa_api.cpp", "fwd.hip", "bwd.hip", "quant.hip", "fwd_fp8.hip", "merge.hip"]
# Sources whose kernels copy tiles with inline-asm LDS-DMA loads: their device
# assembly is checked for the wait states those copies need and for kernels
# that spill registers to scratch (asmcheck.py).
DMA_SOURCES = ["fwd.hip", "bwd.hip", "fwd_fp8.hip"]
# Per-source flags.  The fp8 forward interleaves the P V products of tile j-1
# with the softmax of tile j step by step; machine sinking moves those
# products past the rare-path branch at the end of the tile (their first use
# there is the conditional rescale of O), so that they run back to back with
# no vector work beside them, and raises register pressure (d = 256 then
# spills).
SOURCE_FLAGS = {"fwd_fp8.hip": ["-mllvm", "-disable-machine-sink"]}

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Wno-unused-function",
    # Packed fp32 arithmetic stays off for all device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "unknown target feature" not in l
                     and "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    return obj


def _check_asm(src: str, verbose: bool) -> int:
    """Compile `src`'s device code to assembly and check every LDS-DMA copy;
    returns the number of copies."""
    from exact_tiled_attention_16_amd import asmcheck
    asm = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".s")
    cmd = [_hipcc(), *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), "--cuda-device-only", "-S",
           "-x", "hip", os.path.join(CSRC, src), "-o", asm]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{res.stdout}{res.stderr}")
    with open(asm) as f:
        text = f.read()
    problems = asmcheck.check_text(text)
    if problems:
        raise RuntimeError(f"{src}: LDS-DMA copies without their wait states:\n"
                           + "\n".join(problems[:20]))
    n = asmcheck.copies(text)
    if n == 0:
        raise RuntimeError(f"{src}: no LDS-DMA copies found in the device assembly")
    spills = asmcheck.scratch_kernels(text)
    if spills:
        raise RuntimeError(f"{src}: kernels using scratch (register spills):\n"
                           + "\n".join(f"{k}: {b} bytes" for k, b in spills))
    return n


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, out)


def _program(src, out, verbose):
    tmp = out + ".tmp"
    cmd = [_hipcc(), *COMMON_FLAGS, "-x", "hip", os.path.join(CSRC, src), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                         if "packed-fp32-ops" not in l)
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    os.replace(tmp, out)


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        checks = [ex.submit(_check_asm, s, verbose) for s in DMA_SOURCES]
        rate = ex.submit(_program, RATE_SOURCE, RATE_EXE, verbose)
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES + [PROBE_SOURCE]))
        for c in checks:
            c.result()
        rate.result()
    _link([os.path.join(OBJDIR, os.path.splitext(PROBE_SOURCE)[0] + ".o")], PROBE_LIB, verbose)
    _link(objs[:len(SOURCES)], LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

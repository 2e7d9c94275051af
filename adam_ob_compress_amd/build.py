"""Build libobadam.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libobadam.so")
# (source, extra defines): compiled to objects in parallel, then linked into one library
UNITS = [
    ("ob_compress.hip", ["-DOB_ERR_FMT=0"]),   # fp32 error buffer
    ("ob_compress.hip", ["-DOB_ERR_FMT=1"]),   # bf16
    ("ob_compress.hip", ["-DOB_ERR_FMT=2"]),   # fp16
    ("ob_kernels.hip", []),
    ("ob_noalloc.hip", []),
    ("ob_api.cpp", []),
]
BUILD_DIR = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep packed-fp32 instructions out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def build(verbose: bool = False, extra: list[str] | None = None, out: str | None = None) -> str:
    """Compile every unit (in parallel) and link one shared library; always recompiles."""
    target = out or LIB
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs, objs = [], []
    for i, (src, defs) in enumerate(UNITS):
        obj = os.path.join(BUILD_DIR, f"{i}_{os.path.splitext(src)[0]}.o")
        cmd = [HIPCC, *FLAGS, *defs, *(extra or []), "-c", "-o", obj, os.path.join(CSRC, src)]
        cmd.remove("-shared")
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), cmd))
        objs.append(obj)
    failed = [cmd for p, cmd in procs if p.wait() != 0]
    if failed:
        raise RuntimeError("hipcc failed: " + " ".join(failed[0]))
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", target + ".tmp", *objs]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(target + ".tmp", target)
    return target


PROBE_SRC = os.path.join(PKG, "probe", "ob_probe.hip")
PROBE_LIB = os.path.join(PKG, "probe", "libobprobe.so")


def build_probe(verbose: bool = False) -> str:
    """Compile the measurement probe (a nontemporal copy kernel that bench.py's counter calibration
    runs) into its own library; the optimizer library never loads it."""
    cmd = [HIPCC, *FLAGS, "-o", PROBE_LIB + ".tmp", PROBE_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])

"""Builds libbasa.so for gfx950 from the HIP sources in csrc/ (in-tree).

Usage: python block_sparse_attention_mean_amd/build.py [-v]
(run as a file: importing the package itself needs the built library)
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbasa.so")
PEAK_SRC = os.path.join(HERE, "probes", "peak.hip")
PEAK_LIB = os.path.join(HERE, "libbasa_peak.so")   # measured-peak kernels for bench.py only
ARCH = "gfx950"

# Packed fp32 instructions are disabled for all device code: the compiler
# would otherwise form v_pk_* FMAs from plain float code.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ, os.path.basename(src).replace(".hip", ".o"))
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip and link libbasa.so; returns the library path."""
    os.makedirs(OBJ, exist_ok=True)
    sources = sorted(os.path.join(SRC, f) for f in os.listdir(SRC) if f.endswith(".hip"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), sources))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    build_peak(verbose)
    return LIB


def build_peak(verbose: bool = False) -> str:
    """Compile the measured-peak kernels (probes/peak.hip) into libbasa_peak.so."""
    tmp = PEAK_LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-shared", PEAK_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {PEAK_SRC}:\n{res.stderr}")
    os.replace(tmp, PEAK_LIB)
    return PEAK_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Builds libdq.so (HIP kernels + C ABI) for gfx950 in-tree.

    python -m kv_cache_entropy_amd.build

Every source is compiled with hipcc for gfx950 only.  Flags that matter for
bit-exact parity of the encoder: -ffp-contract=off (no fused multiply-add
changes fp32 results), denormals kept, default (correctly rounded) division
and square root.  Packed fp32 instructions are disabled
(-target-feature -packed-fp32-ops).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdq.so")
PROBE = os.path.join(OBJ, "lds_gather_probe")
SOURCES = ["codec.cpp", "encode.hip", "decode.hip", "attention.hip"]
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall",
          "-I", os.path.join(ROOT, "include")]
HIP_ONLY = [f"--offload-arch={ARCH}", "-fno-gpu-flush-denormals-to-zero",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if p and (os.path.sep not in p or os.path.exists(p)):
            return p
    raise RuntimeError("hipcc not found")


def _compile(src: str, verbose: bool) -> str:
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc()] + COMMON
    if src.endswith(".hip"):
        cmd += HIP_ONLY + ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return out


def build(verbose: bool = False) -> str:
    """Compiles every source (always) and links libdq.so."""
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    # the LDS gather microbenchmark (a program of its own, not part of the library)
    probe = [_hipcc(), "-O3", "-std=c++17", "-Wall"] + HIP_ONLY + [
        "-x", "hip", os.path.join(CSRC, "probes", "lds_gather.hip"), "-o", PROBE]
    if verbose:
        print(" ".join(probe), flush=True)
    r = subprocess.run(probe, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for probes/lds_gather.hip:\n{r.stderr}")
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build libmaskgs (the HIP kernels and the C ABI) in-tree for gfx950."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmaskgs.so")
OBJDIR = os.path.join(PKG, "_build")
SOURCES = ["maskgs_api.hip", "maskgs_k24.hip", "maskgs_k48.hip", "maskgs_debug.hip",
           "maskpro_k.hip"]

# -ffp-contract=off: the noise contract fixes every rounding; fused multiply-adds
# appear only where the source writes them.  Packed fp32 instructions are
# disabled for the whole library.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(REPO, "include"), "-I", CSRC, "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compile libmaskgs.so next to this file (always recompiles; the sources
    compile in parallel, then link)."""
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", "0") or 0) or
                                 (os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


PROBE_SRC = os.path.join(PKG, "calib", "roofline_probe.hip")
PROBE = os.path.join(PKG, "calib", "roofline_probe")


def build_probe(verbose: bool = False) -> str:
    """Compile the roofline calibration program (calib/roofline_probe): HBM
    streams and VALU loops of known size, run on its own and under rocprofv3."""
    cmd = [hipcc(), *[f for f in HIPCC_FLAGS if f != "-fPIC"], PROBE_SRC, "-o", PROBE + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(PROBE + ".tmp", PROBE)
    return PROBE


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_probe(verbose=True))

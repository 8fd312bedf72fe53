"""Ahead-of-time build of libepget.so for gfx950 (in-tree, no JIT)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libepget.so")
SOURCES = ["api.hip", "layout.hip", "rows.hip", "hier.hip"]
# bandwidth probes the benchmark compares the kernels with (not the path)
PROBE_LIB = os.path.join(HERE, "libepprobe.so")
PROBE_SOURCES = ["probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Werror=return-type",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the leading scalar kernel arguments (up to 14 dwords) arrive in SGPRs,
    # not through a load at the start of every wave: the decode-sized
    # kernels take their first loads' operands that way
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(lib: str, sources, verbose: bool) -> str:
    tmp = lib + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp, *[os.path.join(CSRC, s) for s in sources]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile libepget.so and the probe library libepprobe.so (always
    recompiles both)."""
    _compile(PROBE_LIB, PROBE_SOURCES, verbose)
    return _compile(LIB, SOURCES, verbose)


if __name__ == "__main__":
    print(build(verbose=True))

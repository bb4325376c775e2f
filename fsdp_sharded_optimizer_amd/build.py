"""Build libzshard.so (the library) and libzsceiling.so (the benchmark's
bandwidth-ceiling kernel, not part of the library's interface) in-tree with
hipcc for gfx950.

    python -m fsdp_sharded_optimizer_amd.build

Flags that matter for the numerics and for gfx950:
  -ffp-contract=off                          no a*b+c fusion: one rounding per operation
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE fp32 division and square root
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                             no packed-fp32 (v_pk_*_f32) instructions
  -fvisibility=hidden                        export only the C ABI (ZS_API in zshard.h)
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libzshard.so")
CEILING_LIB = os.path.join(HERE, "libzsceiling.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def sources(sub: str = "csrc"):
    return sorted(glob.glob(os.path.join(HERE, sub, "*.hip")))


def build(verbose: bool = False) -> str:
    _compile(CEILING_LIB, sources("ceiling"), verbose)
    return _compile(LIB, sources(), verbose)


def _compile(lib: str, srcs, verbose: bool) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = lib + ".tmp"
    cmd = [hipcc, *FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature and says so
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in proc.stderr.splitlines() if noise not in l and "(ignoring feature)" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))

"""Build libqar.so in-tree with hipcc for gfx950.

Flags: -O3; -ffp-contract=off (no fused multiply-add unless written
explicitly); correctly rounded binary32 division; fp32 denormals kept (no
flush-to-zero flag); packed-fp32 instructions disabled."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libqar.so")
SOURCES = [os.path.join(CSRC, "qar_kernels.hip"), os.path.join(CSRC, "qar_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def build(output: str = LIBRARY, extra: list[str] | None = None, verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    tmp = output + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra or []), "-shared", *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(verbose=True))

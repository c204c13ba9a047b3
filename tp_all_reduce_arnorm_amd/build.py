"""Build libarnorm.so (the C ABI of include/arnorm.h) for gfx950 with hipcc, in-tree.

    python -m tp_all_reduce_arnorm_amd.build

The library is written next to this file; tests, smoke() and bench.py load it from
there.  IEEE FP32 throughout: no fast-math, no FP contraction (the kernels write their
one FMA chain explicitly), denormals kept; packed-FP32 instructions are disabled.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libarnorm.so")
SOURCES = [os.path.join(CSRC, "libarnorm.hip")]
HEADERS = [os.path.join(CSRC, n) for n in ("device.hpp", "arnorm_kernels.hpp", "gather_kernels.hpp",
                                           "twoshot_kernels.hpp")] + [
    os.path.join(INCLUDE, "arnorm.h")
]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def build(verbose=True, out=LIB, defines=()):
    """Compile every HIP source into libarnorm.so (always recompiles)."""
    tmp = out + ".tmp"
    cmd = [HIPCC] + FLAGS + [f"-D{d}" for d in defines] + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, out)
    return out


def assembly(out_path, kernel_filter=None):
    """Write the gfx950 assembly of the library (device code only) to ``out_path``."""
    cmd = [HIPCC] + [f for f in FLAGS if f not in ("-shared", "-fPIC")] + [
        "--cuda-device-only", "-S", SOURCES[0], "-o", out_path]
    subprocess.run(cmd, check=True)
    return out_path


if __name__ == "__main__":
    print(build())

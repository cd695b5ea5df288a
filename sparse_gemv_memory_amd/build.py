"""Build libnm_sparse.so from the HIP sources in csrc/ with hipcc for gfx950.

The library is built in-tree (next to this file) so that it travels with the
source tree; nothing is installed.
"""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
# translation units of the library (headers next to them are included)
SRCS = [os.path.join(CSRC, f) for f in ("nm_sparse.hip", "nm_prefill.hip", "nm_calib.hip", "nm_generic.hip")
        if os.path.exists(os.path.join(CSRC, f))]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libnm_sparse.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # keep hipcc from forming packed fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False) -> str:
    """Compile the HIP library (always rebuilds) and return its path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{INCLUDE}", "-o", tmp, *SRCS]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr:
        print(res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

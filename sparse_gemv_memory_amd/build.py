"""Build libnm_sparse.so from the HIP sources in csrc/ with hipcc for gfx950.

The library is built in-tree (next to this file) so that it travels with the
source tree; nothing is installed.  Each translation unit compiles to an
object of its own (in parallel) under _build/, and the objects are linked
into the shared library.
"""

from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJDIR = os.path.join(HERE, "_build")
# translation units of the library (headers next to them are included)
UNITS = ("nm_sparse.hip", "nm_prefill.hip", "nm_calib.hip", "nm_generic.hip")
SRCS = [os.path.join(CSRC, f) for f in UNITS if os.path.exists(os.path.join(CSRC, f))]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libnm_sparse.so")
ARCH = "gfx950"

# Keep hipcc from forming packed fp32 VALU ops (v_pk_*_f32) in device code.
# The clang driver cannot forward -Xclang options to the device pass alone
# (-Xarch_device refuses them), and a per-function target attribute stops
# the HIP header functions (shuffles, exp) from being inlined, so the feature
# reaches the host pass too, which ignores it with one warning per unit.
NO_PACKED_FP32 = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
HOST_FEATURE_WARNING = "'-packed-fp32-ops' is not a recognized feature"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    *NO_PACKED_FP32,
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    # the host pass's notice about the device-only feature is expected
    return "\n".join(l for l in res.stderr.splitlines() if HOST_FEATURE_WARNING not in l)


def _compile(src: str) -> tuple:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    return obj, _run([hipcc(), *HIPCC_FLAGS, f"-I{INCLUDE}", "-c", src, "-o", obj])


def build(verbose: bool = False) -> str:
    """Compile the HIP library (always rebuilds) and return its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    workers = max(1, min(len(SRCS), os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        results = list(ex.map(_compile, SRCS))
    tmp = LIB + ".tmp"
    log = _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
                *[obj for obj, _ in results]])
    if verbose:
        for _, msg in results + [(None, log)]:
            if msg.strip():
                print(msg)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Two builds, each checked by running an existing CPU test file against it in a
child process with the matching sanitizer runtime preloaded:

* the oracle (oracle/nm_oracle.c) built by gcc with ASan + UBSan, running
  every pin of tests/test_oracle_pins.py (NM_ORACLE_LIB selects the build);
* the HIP library built by hipcc with the sanitizers on its host pass only
  (each -fsanitize= behind -Xarch_host; device code is built as usual and
  never runs here), running the C-ABI argument checks of
  tests/test_capi_cpu.py (NM_CAPI_LIB selects the build).

UBSan stops at the first finding (-fno-sanitize-recover), ASan at its first
report; leak checking is off because the Python interpreter itself keeps
allocations alive at exit.
"""

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_gemv_memory_amd", "csrc")
UNITS = ("nm_sparse.hip", "nm_prefill.hip", "nm_calib.hip", "nm_generic.hip")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run_tests(test_file, env_extra):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", test_file)],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    log = res.stdout + res.stderr
    assert "Sanitizer" not in log and "runtime error:" not in log, log[-4000:]
    assert res.returncode == 0, log[-4000:]
    return log


def _loaded_in_child(probe, env_extra, needle):
    """True if a child interpreter with env_extra maps a file whose path holds
    needle after running probe."""
    env = dict(os.environ, **SAN_ENV, **env_extra)
    code = f"{probe}\nprint(open('/proc/self/maps').read().count({needle!r}) > 0)"
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    return res.stdout.strip().endswith("True")


def test_oracle_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not (shutil.which("gcc") and asan and ubsan):
        pytest.skip("gcc with the ASan / UBSan runtimes is not available")
    lib = str(tmp_path / "libnm_oracle_asan.so")
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fopenmp", "-shared", "-fPIC", "-std=c99",
                    "-Wall", "-o", lib, os.path.join(ROOT, "oracle", "nm_oracle.c"), "-lm"],
                   check=True)
    env = {"NM_ORACLE_LIB": lib, "LD_PRELOAD": f"{asan}:{ubsan}"}
    assert _loaded_in_child("import oracle; oracle._load()", env, "libnm_oracle_asan.so")
    log = _run_tests("test_oracle_pins.py", env)
    assert " passed" in log


def _clang_asan_runtime():
    pats = ["/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so",
            "/opt/rocm/llvm/lib/clang/*/lib/x86_64-unknown-linux-gnu/libclang_rt.asan.so"]
    for pat in pats:
        hits = sorted(glob.glob(pat))
        if hits:
            return hits[-1]
    return None


def test_hip_host_code_under_asan_and_ubsan(tmp_path):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    runtime = _clang_asan_runtime()
    if not (os.path.exists(hipcc) and runtime):
        pytest.skip("hipcc or clang's ASan runtime is not available")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    flags = ["--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             *host_san, "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-g",
             f"-I{os.path.join(ROOT, 'include')}"]
    procs, objs = [], []
    for unit in UNITS:
        obj = str(tmp_path / (unit + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([hipcc, *flags, "-c", os.path.join(CSRC, unit), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out, _ = p.communicate(timeout=900)
        assert p.returncode == 0, out
    lib = str(tmp_path / "libnm_sparse_asan.so")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *host_san, "-shared-libsan",
                    "-o", lib, *objs], check=True, capture_output=True)
    env = {"NM_CAPI_LIB": lib, "LD_PRELOAD": runtime}
    probe = ("import ctypes, os; from sparse_gemv_memory_amd import native; "
             "native.declare(ctypes.CDLL(os.environ['NM_CAPI_LIB']))")
    assert _loaded_in_child(probe, env, "libnm_sparse_asan.so")
    log = _run_tests("test_capi_cpu.py", env)
    assert " passed" in log

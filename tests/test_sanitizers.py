"""CPU sanitizer runs (no GPU): the oracle under AddressSanitizer and
UndefinedBehaviorSanitizer running its pins, and the library's host code
(argument validation, launch planning, workspace layout, the adaptive-length
controller) under the same sanitizers running the ABI tests.  Each build
goes to a temporary directory and each run is a child process with the
sanitizer runtime preloaded; a planted out-of-bounds write first shows that
the runtime really reports."""
import glob
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "proposal_sv_verify_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}
ORACLE_PINS = ["tests/test_oracle_greedy.py", "tests/test_oracle_rejection.py",
               "tests/test_oracle_tree_ngram.py", "tests/test_oracle_suffix.py",
               "tests/test_oracle_adaptive.py"]


def _gcc_runtime():
    path = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return path


def _clang_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits or not os.path.exists(HIPCC):
        pytest.skip("ROCm's clang AddressSanitizer runtime or hipcc is not installed")
    return hits[-1]


def _run(cmd, preload, extra_env=None, timeout=600):
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=preload, **(extra_env or {}))
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)


def test_planted_overflow_is_reported(tmp_path):
    """The harness is live: a one-past-the-end write in a library built with
    the oracle's sanitizer flags makes the child process fail with a report."""
    rt = _gcc_runtime()
    src = tmp_path / "bad.c"
    src.write_text("#include <stdlib.h>\nint bad(int n) { int *a = malloc(n * sizeof(int));"
                   " a[n] = 1; int r = a[0]; free(a); return r; }\n")
    so = str(tmp_path / "libbad.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-shared", "-fPIC", "-o", so, str(src)])
    r = _run([sys.executable, "-c", "import ctypes; ctypes.CDLL(%r).bad(4)" % so], rt)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr


def test_oracle_pins_under_asan_ubsan(tmp_path):
    rt = _gcc_runtime()
    so = str(tmp_path / "liboracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer", "-shared", "-fPIC", "-I",
                           os.path.dirname(oracle.__file__), "-o", so,
                           os.path.join(os.path.dirname(oracle.__file__), "oracle.c"), "-lm"])
    r = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"]
             + ORACLE_PINS, rt, {"SPECVERIFY_ORACLE": so})
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr


def test_library_host_code_under_asan_ubsan(tmp_path):
    rt = _clang_runtime()
    so = str(tmp_path / "libspecverify_san.so")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC] + sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + \
          ["-o", so]
    subprocess.check_call(cmd, stderr=subprocess.DEVNULL)
    r = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
              "tests/test_abi.py", "tests/test_adaptive.py"], rt, {"SPECVERIFY_LIBRARY": so})
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr

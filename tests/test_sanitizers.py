"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

1. The oracle: oracle/dust_oracle.c built with gcc's sanitizers, and every
   oracle pin and oracle property test run against that build.
2. libdust's host code: every source built as usual for gfx950 but with the
   host side instrumented (device code is never run here), and the C ABI's
   host-side checks (tests/test_abi.py and the ABI property tests, which send
   random and extreme sizes, enums and parameters) run against that build.

Each run is a child Python process with the sanitizer runtime preloaded; any
report (an out-of-bounds access, a signed overflow, an invalid enum load, ...)
aborts it.  Builds land in _build/sanitize/ and are redone when a source is
newer.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from util import ROOT

SAN_DIR = os.path.join(ROOT, "_build", "sanitize")
KINDS = ("address", "undefined")
REPORT_MARKS = ("ERROR: AddressSanitizer", "runtime error:", "SUMMARY: UndefinedBehaviorSanitizer")
ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _stale(out, sources):
    return not os.path.exists(out) or any(os.path.getmtime(s) > os.path.getmtime(out)
                                          for s in sources)


def _run(cmd, preload, extra_env, timeout=900):
    env = dict(os.environ)
    env.update(ENV)
    env.update(extra_env)
    env["LD_PRELOAD"] = preload
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    out = res.stdout + res.stderr
    reports = [m for m in REPORT_MARKS if m in out]
    assert res.returncode == 0 and not reports, out[-6000:]
    return out


def _gcc_runtime():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return path


def _clang_runtime():
    clang = "/opt/rocm/llvm/bin/clang"
    if not os.path.exists(clang):
        pytest.skip("the ROCm clang is not installed")
    path = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                          capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    return path


def test_oracle_under_sanitizers():
    runtime = _gcc_runtime()
    src = os.path.join(ROOT, "oracle", "dust_oracle.c")
    lib = os.path.join(SAN_DIR, "libdust_oracle.so")
    os.makedirs(SAN_DIR, exist_ok=True)
    if _stale(lib, [src]):
        san = "-fsanitize=" + ",".join(KINDS)
        subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", san,
                               "-fno-sanitize-recover=undefined", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", lib, src, "-lm"])
    tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    tests.append(os.path.join(ROOT, "tests", "test_properties.py"))
    prog = ("import sys, oracle, pytest\n"
            f"assert oracle._load()._name == {lib!r}\n"
            f"sys.exit(pytest.main({tests!r} + ['-q', '-s', '-x', '-p', 'no:cacheprovider', "
            "'-m', 'not gpu', '-k', 'not answers and not queries and not status']))\n")
    out = _run([sys.executable, "-c", prog], runtime, {"DUST_ORACLE_LIB": lib})
    assert " passed" in out


def test_abi_host_checks_under_sanitizers():
    runtime = _clang_runtime()
    from activation_perturbation_estimator_amd import build as b
    lib = os.path.join(SAN_DIR, "libdust.so")
    sources = [os.path.join(b.CSRC, s) for s in b.SOURCES]
    sources += glob.glob(os.path.join(b.CSRC, "*.hpp")) + [os.path.join(b.INCLUDE, "dust.h")]
    if _stale(lib, sources):
        flags = []
        for k in KINDS:  # host side only: the device code is built as usual
            flags += ["-Xarch_host", "-fsanitize=" + k]
        flags += ["-Xarch_host", "-fno-sanitize-recover=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
        b.build(extra_flags=flags, out=lib, build_dir=os.path.join(SAN_DIR, "obj"))
    tests = [os.path.join(ROOT, "tests", "test_abi.py"),
             os.path.join(ROOT, "tests", "test_properties.py")]
    prog = ("import sys\n"
            f"sys.path.insert(0, {os.path.join(ROOT, 'tests')!r})\n"
            "from activation_perturbation_estimator_amd import _lib\n"
            f"_lib.LIB_PATH = {lib!r}\n"
            "import pytest\n"
            f"sys.exit(pytest.main({tests!r} + ['-q', '-s', '-x', '-p', 'no:cacheprovider', "
            "'-m', 'not gpu', '-k', 'not sum_to_zero and not recurrence and not linear_in']))\n")
    out = _run([sys.executable, "-c", prog], runtime, {})
    assert " passed" in out

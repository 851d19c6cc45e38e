"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Three pieces of host code run here with -fsanitize=address,undefined and
-fno-sanitize-recover=all, so that any undefined behaviour or bad access
aborts the run:
  * the launch planners and argument rules (nm_plan.h, nm_rules.h), swept by
    tests/sanitize/plan_sweep.cpp over shapes, batches, CU counts and the
    tuning overrides, every plan checked against what its kernel assumes;
  * the C entry points' checks (nmapi.cpp), linked with a stand-in for the
    kernel side (tests/sanitize/launch_stub.cpp) that checks the launch
    preconditions: random calls (tests/sanitize/abi_fuzz.cpp), and the whole
    of tests/test_abi.py against that build;
  * the CPU oracle (oracle/nm_oracle.c): its pins, and the planted-mistake
    copies, against sanitized builds.
Python runs with the sanitizer runtime preloaded (the library is built as a
shared object); leak checking is off, since the interpreter frees little at
exit.  Device code is not involved: it does not run without a GPU.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
CSRC = os.path.join(ROOT, "sparse_matrix_vector_amd", "csrc")
SAN = os.path.join(TESTS, "sanitize")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1", "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


pytestmark = pytest.mark.skipif(shutil.which("g++") is None or _runtime("libasan.so") is None,
                                reason="needs g++ with the AddressSanitizer runtime")


def _build(cmd):
    proc = subprocess.run(cmd, capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr


def _run(cmd, preload=False, timeout=600):
    env = dict(os.environ, **SAN_ENV)
    env["PYTHONPATH"] = os.pathsep.join([ROOT, TESTS])
    if preload:
        env["LD_PRELOAD"] = _runtime("libasan.so")
    proc = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout, cwd=ROOT)
    out = proc.stdout + proc.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    return proc, out


def _cxx(out, *sources, shared=False):
    cmd = ["g++", "-std=c++17", "-Wall", "-Wextra", *SAN_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *sources, "-o", out]
    if shared:
        cmd[1:1] = ["-fPIC", "-shared"]
    _build(cmd)
    return out


def test_planners_and_rules_under_sanitizers(tmp_path):
    exe = _cxx(str(tmp_path / "plan_sweep"), os.path.join(SAN, "plan_sweep.cpp"))
    env_clean = {k: v for k, v in os.environ.items() if not k.startswith("NMSPMV_")}
    proc = subprocess.run([exe], capture_output=True, text=True, env=dict(env_clean, **SAN_ENV), timeout=600)
    out = proc.stdout + proc.stderr
    assert proc.returncode == 0, out[-4000:]
    assert "plans checked" in out


def test_entry_point_checks_fuzzed_under_sanitizers(tmp_path):
    exe = _cxx(str(tmp_path / "abi_fuzz"), os.path.join(SAN, "abi_fuzz.cpp"), os.path.join(SAN, "launch_stub.cpp"),
               os.path.join(CSRC, "nmapi.cpp"))
    proc, out = _run([exe, "200000"])
    assert proc.returncode == 0, out[-4000:]


def test_abi_suite_under_sanitizers(tmp_path):
    """tests/test_abi.py against nmapi.cpp built with sanitizers: the same
    entry points and checks as the product library, with the kernel side
    replaced by the stub, which none of those calls may reach."""
    lib = _cxx(str(tmp_path / "libnmspmv_checks.so"), os.path.join(CSRC, "nmapi.cpp"),
               os.path.join(SAN, "launch_stub.cpp"), shared=True)
    code = ("import sys, ctypes, pytest\n"
            "import sparse_matrix_vector_amd._lib as L\n"
            "L.LIB_PATH = sys.argv[1]\n"
            "rc = pytest.main([sys.argv[2], '-q', '-x', '-p', 'no:cacheprovider'])\n"
            "n = ctypes.CDLL(sys.argv[1]).nmtest_launches()\n"
            "print('launches', n)\n"
            "sys.exit(rc or (n != 0))\n")
    proc, out = _run([sys.executable, "-c", code, lib, os.path.join(TESTS, "test_abi.py")], preload=True)
    assert proc.returncode == 0, out[-4000:]
    assert "launches 0" in out and " passed" in out


def _oracle_lib(tmp_path, source, name):
    lib = str(tmp_path / name)
    _build(["gcc", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", *SAN_FLAGS, source, "-o", lib, "-lm"])
    return lib


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = _oracle_lib(tmp_path, os.path.join(ROOT, "oracle", "nm_oracle.c"), "liboracle_san.so")
    code = ("import sys, pytest, oracle\n"
            "oracle.use_library(sys.argv[1])\n"
            "sys.exit(pytest.main([sys.argv[2], '-q', '-x', '-p', 'no:cacheprovider']))\n")
    proc, out = _run([sys.executable, "-c", code, lib, os.path.join(TESTS, "test_oracle_pins.py")], preload=True)
    assert proc.returncode == 0, out[-4000:]
    assert " passed" in out


def test_oracle_mutants_caught_under_sanitizers(tmp_path):
    """Every planted mistake of tests/test_oracle_mutants.py, built with the
    sanitizers: each copy must still fail a pin (or abort on a sanitizer
    report, which also counts as caught); the real oracle passes them all."""
    import test_oracle_mutants as M
    text = open(M.SRC).read()
    code = ("import sys, oracle, test_oracle_mutants as t; oracle.use_library(sys.argv[1]); "
            "f = t._failing_pins(); print(f); sys.exit(1 if f else 0)")
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=_runtime("libasan.so"), PYTHONPATH=os.pathsep.join([ROOT, TESTS]))

    def caught(mutant):
        name, old, new = mutant
        assert text.count(old) == 1, name
        src = tmp_path / f"{name}.c"
        src.write_text(text.replace(old, new))
        lib = _oracle_lib(tmp_path, str(src), f"lib{name}.so")
        proc = subprocess.run([sys.executable, "-c", code, lib], capture_output=True, text=True, env=env, timeout=300)
        return name, proc.returncode != 0

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
        for name, ok in pool.map(caught, M.MUTANTS):
            assert ok, f"planted mistake {name} passed every pin under the sanitizers"


PLANTED = r"""
#include <limits.h>
#include <stdlib.h>
int planted_heap_overflow(int n) { int* p = malloc(4 * sizeof(int)); p[n] = 1; int v = p[0]; free(p); return v; }
int planted_signed_overflow(int a) { return a + 1; }
"""


@pytest.mark.parametrize("call,reports", [("planted_heap_overflow(4)", ("heap-buffer-overflow", "insufficient space")),
                                          ("planted_signed_overflow(2147483647)", ("signed integer overflow",))])
def test_sanitizers_are_live(tmp_path, call, reports):
    """The set-up above would pass vacuously if the instrumentation or the
    preloaded runtime were missing: a planted overflow must be reported."""
    src = tmp_path / "planted.c"
    src.write_text(PLANTED)
    lib = _oracle_lib(tmp_path, str(src), "libplanted.so")
    code = f"import ctypes, sys; lib = ctypes.CDLL(sys.argv[1]); lib.{call}"
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=_runtime("libasan.so"))
    proc = subprocess.run([sys.executable, "-c", code, lib], capture_output=True, text=True, env=env, timeout=120)
    assert proc.returncode != 0 and any(r in proc.stderr for r in reports), proc.stderr[-2000:]

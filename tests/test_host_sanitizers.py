"""The library's host layer (argument validation, aliasing checks, tree
parsing and descriptor packing: csrc/api.cpp and csrc/tree_meta.cpp) built
with AddressSanitizer and UndefinedBehaviorSanitizer, linked with stand-in
launchers instead of the GPU kernels (tests/host_check/stub_launchers.cpp),
and the C-ABI test module run against that build in a child process.

The build uses the host compiler only (g++; no GPU code is compiled), so it
runs on any machine.  Every sanitizer report aborts the child, so a report is
a failed test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_deltanet_tree_03_amd", "csrc")
OUT_DIR = os.path.join(ROOT, "_build", "hostcheck")
LIB = os.path.join(OUT_DIR, "libtreewy_hostcheck.so")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


def _build():
    os.makedirs(OUT_DIR, exist_ok=True)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fPIC", "-shared",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           "-I" + CSRC, os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "tree_meta.cpp"),
           os.path.join(ROOT, "tests", "host_check", "stub_launchers.cpp"), "-o", LIB]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout


def test_abi_tests_under_asan_and_ubsan():
    _build()
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], stdout=subprocess.PIPE,
                          text=True).stdout.strip()
    assert os.path.isabs(asan) and os.path.exists(asan), "libasan.so not found"
    env = dict(os.environ)
    # the sanitizer runtime must come first; keep whatever the environment
    # already preloads after it
    env["LD_PRELOAD"] = " ".join(x for x in (asan, os.environ.get("LD_PRELOAD", "")) if x)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["TREEWY_LIB"] = LIB
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=600)
    tail = "\n".join(r.stdout.splitlines()[-30:])
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stdout and "runtime error" not in r.stdout, tail
    # the stand-in launchers were loaded: the tests that need them ran
    assert " skipped" not in r.stdout.splitlines()[-1], tail

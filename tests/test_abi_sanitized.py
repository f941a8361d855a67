"""The C ABI's host-side argument checking (csrc/mx_api.cpp) under
AddressSanitizer and UndefinedBehaviorSanitizer.

mx_api.cpp is compiled with g++ (host code only, no HIP compiler involved)
and linked with tests/sanitize/launch_stubs.cpp, whose launchers return
success without touching their pointers. tests/test_abi_cpu.py then runs
against that library in a subprocess with the ASan runtime preloaded (the
Python interpreter itself is not instrumented): every validation case, the
size queries, the per-thread error messages and the exported-symbol check.
The cases whose answers come from the GPU-side planner (plan names,
workspace sizes) are left out, since the stubs do not plan. Any sanitizer
report aborts the subprocess and fails the test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_scaled_precision_mx_amd", "csrc")


def _gcc_runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("g++") is None or _gcc_runtime("libasan.so") is None,
                    reason="needs g++ with the AddressSanitizer runtime")
def test_abi_checks_under_sanitizers(tmp_path):
    lib = str(tmp_path / "libmx_sanitized.so")
    build = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-shared", "-fPIC", "-Wl,--no-undefined", "-D__HIP_PLATFORM_AMD__",
             "-I/opt/rocm/include", "-I" + CSRC, os.path.join(CSRC, "mx_api.cpp"),
             os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"), "-o", lib]
    r = subprocess.run(build, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]

    runner = ("import sys; sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r}); "
              "from block_scaled_precision_mx_amd import _lib; _lib.LIB_PATH = {lib!r}; import pytest; "
              "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu', "
              "'-k', 'not plan and not bench_workloads', {test!r}]))").format(
        root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib, test=os.path.join(ROOT, "tests", "test_abi_cpu.py"))
    env = dict(os.environ)
    env["LD_PRELOAD"] = _gcc_runtime("libasan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-c", runner], env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    report = (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert r.returncode == 0, report
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, report
    assert " passed" in r.stdout, report

"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* The oracle (oracle/oracle.c) is compiled with gcc -fsanitize=address,
  undefined and its pin and invariant tests run against that build.
* The library is compiled with host-side sanitizers (device code unchanged)
  and the tests of its host code run against it: the tree schedule
  (tree_plan.cpp), the junction symbolic analysis (junction_plan.cpp) and the
  C-ABI argument checks (abi.cpp).  With no GPU here, calls that pass their
  argument checks stop at the first HIP call with an error status, so the
  error paths (plan clean-up included) run too.

Each run is a child process with the matching sanitizer runtime preloaded
(the Python interpreter itself is not instrumented).  Any sanitizer report
aborts the child, and the test fails.
"""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

HERE = os.path.dirname(os.path.abspath(__file__))
SAN_DIR = os.path.join(ROOT, "_build", "sanitize")
SAN_ENV = {
    "ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=1:"
                    "halt_on_error=1",
    "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    "OMP_NUM_THREADS": "2",
}


def _run(which, so, runtime, files):
    env = dict(os.environ, LD_PRELOAD=runtime, **SAN_ENV)
    r = subprocess.run([sys.executable, os.path.join(HERE, "sanitize_child.py"), which, so]
                       + files, env=env, capture_output=True, text=True, timeout=1500)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def _gcc_runtime(name):
    return subprocess.check_output(["gcc", "-print-file-name=" + name], text=True).strip()


@pytest.mark.timeout(1800)
def test_oracle_under_asan_ubsan():
    os.makedirs(SAN_DIR, exist_ok=True)
    so = os.path.join(SAN_DIR, "liboracle_asan.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-fPIC",
                           "-shared", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", "-fno-fast-math", "-o", so,
                           os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    _run("oracle", so, _gcc_runtime("libasan.so"),
         ["test_oracle_pins.py", "test_oracle_invariants.py", "test_oracle_vjp.py",
          "test_oracle_shared.py", "test_oracle_nonsym.py", "test_oracle_junction.py"])


@pytest.mark.timeout(1800)
def test_library_host_code_under_asan_ubsan():
    import glob
    from sparse_spd_selected_amd import buildlib
    so = os.path.join(SAN_DIR, "libselinv_asan.so")
    flags = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
             "-fno-omit-frame-pointer"]
    buildlib.build(out=so, build_dir=os.path.join(SAN_DIR, "obj"), host_flags=flags)
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rt:
        pytest.skip("clang AddressSanitizer runtime not found")
    _run("library", so, rt[0], ["test_abi.py", "test_tree_schedule.py",
                                "test_junction_symbolic.py"])

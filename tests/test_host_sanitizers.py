"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The C ABI's host side -- argument checks, the index maps, ring plans and
launch planning (ra_api.cpp) -- is rebuilt with both sanitizers (host
compilation only; the kernels are the normal objects) and the CPU tests of
that code (tests/test_plan.py, tests/test_abi.py) run against it in a child
process with the ASan runtime preloaded.  Any out-of-bounds access, use after
free or undefined behaviour in those paths aborts the child.  CPU only: no
test in those files launches a kernel.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_ra_build", os.path.join(ROOT, "ring_attention_blockwise_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_plan_and_abi_tests_pass_under_asan_and_ubsan():
    b = _build_module()
    runtime = b.asan_runtime()
    if runtime is None or not os.path.exists(b.hipcc()):
        pytest.skip("no hipcc or no ASan runtime")
    lib = b.build_sanitized()
    # the instrumentation is really in the host object
    nm = subprocess.run(["nm", os.path.join(os.path.dirname(lib), "ra_api.o")], capture_output=True, text=True)
    assert "__asan_report" in nm.stdout and "__ubsan_handle" in nm.stdout
    env = dict(os.environ, RA_LIBRARY=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    code = ("import ctypes, sys; import ring_attention_blockwise_amd as ra; "
            "assert ra.LIB_PATH == sys.argv[1]; ctypes.CDLL(None)['__asan_init']; print('sanitized', ra.LIB_PATH)")
    r = subprocess.run([sys.executable, "-c", code, lib], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0 and "sanitized" in r.stdout, r.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        "tests/test_plan.py", "tests/test_abi.py"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert r.returncode == 0, out[-3000:]
    assert " passed" in r.stdout

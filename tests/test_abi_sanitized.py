"""The C ABI's host-side checks under AddressSanitizer and UndefinedBehaviorSanitizer.

api.hip (every argument check of the boundary) is built with both sanitisers on
its host code (build.py's build_sanitized), and the CPU ABI tests run against
that library in a child process with clang's shared ASan runtime loaded first.
Any sanitiser report, or a failing test, fails this test.  Nothing here touches
a GPU: the ABI tests stop at the host checks.
"""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "q4nx_build_san", os.path.join(ROOT, "gemm_q4nx_chunk_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_abi_checks_are_clean_under_asan_and_ubsan():
    b = _build_module()
    objs = [os.path.join(b.OBJDIR, s.replace(".hip", ".o")) for s in b.SOURCES if s != "api.hip"]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("the library's objects are not built")
    rt = b.asan_runtime()
    if not os.path.exists(rt):
        pytest.skip("no shared ASan runtime next to the compiler")
    lib = b.build_sanitized()
    pre = os.environ.get("LD_PRELOAD", "")
    env = dict(os.environ, LD_PRELOAD=rt + (":" + pre if pre else ""), Q4NX_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    child = (
        "import sys, pytest\n"
        f"rc = pytest.main([{os.path.join(ROOT, 'tests', 'test_abi_host.py')!r}, '-q', '-p', 'no:cacheprovider'])\n"
        "maps = open('/proc/self/maps').read()\n"
        f"print('sanitised library loaded:', {lib!r} in maps and 'libclang_rt.asan' in maps)\n"
        "sys.exit(int(rc))\n")
    r = subprocess.run([sys.executable, "-c", child], env=env, cwd=ROOT, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert "Sanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "sanitised library loaded: True" in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]

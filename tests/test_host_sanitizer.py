"""The C ABI layer's host code (validation, sizes, workspace layout) under AddressSanitizer
and UndefinedBehaviorSanitizer: a host-only build of psa_api.cpp (device launchers stubbed)
runs every host ABI test in a child process with the sanitizer runtime preloaded. Any
sanitizer report fails the child (halt on error) and so this test. No GPU is used."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def hostcheck_lib():
    sys.path.insert(0, os.path.join(ROOT, "level_pooled_kv_amd"))
    try:
        import build_hostcheck
    finally:
        sys.path.pop(0)
    lib = build_hostcheck.build(verbose=False)
    return lib, build_hostcheck.asan_runtime()


def test_host_abi_tests_clean_under_sanitizers(hostcheck_lib):
    lib, asan = hostcheck_lib
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan" in syms and "__ubsan" in syms, "the host-check build is not instrumented"
    env = dict(os.environ, PSA_LIBRARY=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out

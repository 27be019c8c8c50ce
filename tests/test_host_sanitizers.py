"""The library's host code (argument validation, sizing, workspace carve-up,
launch sequencing) under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the host-sanitizer variant of libspade.so (device code unchanged),
then runs the C-ABI boundary tests in a child process that preloads the ASan
runtime and loads that build through SPADE_LIB.  Any sanitizer report aborts
the child, which fails this test.  Nothing here touches a GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "input_adaptive_block_amd"))


def _asan_runtime():
    r = subprocess.run(["/opt/rocm/lib/llvm/bin/clang", "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isfile(path) else None


def test_boundary_checks_under_host_sanitizers():
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("no ASan runtime in this toolchain")
    import importlib.util
    spec = importlib.util.spec_from_file_location("_spade_build", os.path.join(ROOT, "input_adaptive_block_amd",
                                                                               "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    lib = b.build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=runtime, SPADE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    child = (
        "import sys, pytest\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "import input_adaptive_block_amd as spade\n"
        "maps = open('/proc/self/maps').read()\n"
        f"assert {lib!r} in maps, 'sanitizer build not loaded'\n"
        f"sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', {os.path.join(ROOT, 'tests', 'test_boundary_cpu.py')!r}]))\n"
    )
    r = subprocess.run([sys.executable, "-c", child], env=env, cwd="/tmp", capture_output=True, text=True,
                       timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout

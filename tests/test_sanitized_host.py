"""The host code of libpkv (descriptor validation and launch planning of the
kernel entry points, the prefix cache and the radix tree) under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

The build's sanitizer option (`python -m prefix_reuse_amd.build --sanitize`;
here into a temporary directory) builds libpkv_san.so: device code unchanged,
every host object instrumented. The host test files then run
against it in a child process with the clang ASan runtime preloaded. Any
out-of-bounds access, use after free or undefined behaviour aborts the child
and fails this test. (Leak detection is off: the Python interpreter itself
does not free everything at exit.)"""
from __future__ import annotations

import importlib.util
import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent


def _build_module():
    spec = importlib.util.spec_from_file_location("_pkv_build", ROOT / "prefix_reuse_amd" / "build.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.timeout(900)
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    b = _build_module()
    lib = b.build_sanitized(tmp_path)
    runtime = b.asan_runtime()
    assert Path(runtime).exists(), runtime
    env = dict(os.environ, PKV_LIBRARY=str(lib), LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          "tests/test_prefix_index_host.py", "tests/test_abi_host.py"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=800)
    tail = "\n".join((res.stdout + res.stderr).splitlines()[-30:])
    print(tail)
    assert res.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr

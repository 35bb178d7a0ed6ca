"""The C ABI from plain C: tests/c_abi_consumer.c (C99, built with -pedantic
-Werror against include/pkv.h and include/pkv_prefix.h only) checks status
codes, error messages, the chain-hash prefix cache and the radix tree with no
GPU call."""
import subprocess

import pytest

from prefix_reuse_amd import build as pkv_build


def consumer():
    """The built consumer program (built here if the library build left none)."""
    path = pkv_build.C_CONSUMER_PATH
    if not path.exists():
        pkv_build.build_c_consumer()
    return path


def test_c_consumer_builds_strict_c99():
    # rebuilt here from the committed source: a C99 compiler accepts the headers with every warning an error
    assert pkv_build.build_c_consumer().exists()


def test_c_consumer_host_calls():
    res = subprocess.run([str(consumer()), "host"], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stderr
    assert res.stdout.strip() == "host ok"


def test_c_consumer_rejects_bad_usage():
    res = subprocess.run([str(consumer())], capture_output=True, text=True, timeout=60)
    assert res.returncode == 2 and "usage" in res.stderr


if __name__ == "__main__":
    raise SystemExit(pytest.main([__file__, "-q"]))

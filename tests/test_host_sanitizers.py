"""The C ABI's host side under AddressSanitizer and UndefinedBehavior-
Sanitizer: every library source compiled with host-side sanitizers and
linked with a driver (kv_cache_mixed_top_amd/sanitize/abi_host_check.cpp)
that runs every entry point's argument checks, size queries and launch
planning with no GPU visible.  A sanitizer report or a failed check fails
the test."""
import os
import shutil

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("/opt/rocm/bin/hipcc") is None, reason="needs hipcc")
def test_abi_host_code_under_asan_ubsan():
    san = pytest.importorskip("kv_cache_mixed_top_amd.sanitize")
    san.build_checker()
    p = san.run_checker()
    assert p.returncode == 0, p.stdout[-4000:]
    assert "abi host checks passed" in p.stdout
    assert "ERROR: AddressSanitizer" not in p.stdout and "runtime error" not in p.stdout

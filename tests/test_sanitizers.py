"""Host code under AddressSanitizer and UBSan (CPU only).

The oracle's C attention and the host side of libkvhier.so are rebuilt with
the sanitizers, and the CPU suites that reach them run in child processes with
the matching sanitizer runtime preloaded:
  - the oracle's pins (every call of the C attention, brute-force and closed
    forms) on the gcc build of ``attn_ref.c``;
  - the C ABI checks (every declared symbol, rejected configurations, null
    handles, creation that fails after its checks and frees what it built) on
    the hipcc build with host-side sanitizers.
Any sanitizer report aborts the child, which fails the test.
"""
import os
import subprocess
import sys

import pytest

from tests.conftest import ROOT

ORACLE_SUITES = ["tests/test_oracle_pins.py", "tests/test_tail_oracle.py", "tests/test_compress_oracle.py",
                 "tests/test_reuse_oracle.py", "tests/test_residency_oracle.py"]


def _run(env_extra, args, timeout):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"      # the interpreter keeps memory by design
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *args]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


def test_oracle_attention_under_asan_ubsan():
    import oracle.native as native
    lib = native.build_sanitized()
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("gcc AddressSanitizer runtime not available")
    out = _run({"LD_PRELOAD": asan, "ORACLE_ATTN_LIBRARY": lib}, ORACLE_SUITES, 900)
    assert " passed" in out


def test_library_host_code_under_asan_ubsan():
    from hierarchical_sparse_kv_verify_amd import build
    lib = build.build_sanitized()
    rt = build.sanitizer_runtime()
    out = _run({"LD_PRELOAD": rt, "KVHIER_LIBRARY": lib, "KVHIER_EXPECT_SANITIZED": "1"},
               ["tests/test_abi.py"], 900)
    assert " passed" in out

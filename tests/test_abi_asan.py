"""The C ABI's host code under AddressSanitizer: tests/test_abi.py run against the copy
of the library whose host code is built with -fsanitize=address
(``python -m gated_delta_rule_39_amd.build --asan``; ``__graft_entry__.build()`` builds it
too), in a child process with the sanitizer runtime preloaded.  CPU only: the ABI tests
validate arguments and launch nothing.  Skipped when the copy or the runtime is absent."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from gated_delta_rule_39_amd.build import ASAN_LIB  # noqa: E402


def _asan_runtime():
    for clang in ("/opt/rocm/llvm/bin/clang", "clang"):
        try:
            out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                                 capture_output=True, text=True, timeout=60).stdout.strip()
        except (OSError, subprocess.SubprocessError):
            continue
        if out and os.path.isabs(out) and os.path.exists(out):
            return out
    return None


def test_abi_tests_pass_under_address_sanitizer():
    rt = _asan_runtime()
    if not os.path.exists(ASAN_LIB) or rt is None:
        pytest.skip("host-sanitized libkda.so or the ASan runtime not available")
    with open(ASAN_LIB, "rb") as fh:
        assert b"__asan_report_load" in fh.read(), "the copy is not instrumented"
    env = dict(os.environ, KDA_LIB_PATH=ASAN_LIB, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=0")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                          "-p", "no:cacheprovider", "tests/test_abi.py"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    report = res.stdout[-4000:] + res.stderr[-4000:]
    assert "AddressSanitizer" not in res.stderr, report
    assert res.returncode == 0, report
    assert " passed" in res.stdout, report

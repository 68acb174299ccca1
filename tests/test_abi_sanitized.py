"""The C ABI's host-side checks (tests/test_abi.py) run again, in a child
process, against a copy of the library whose host code is built with
AddressSanitizer and UndefinedBehaviorSanitizer (every finding fatal): an
out-of-bounds access, a use after free, an integer overflow or an invalid
enum load in the argument checks, size queries or caches fails this test
with the sanitizer's report.  CPU only: no call reaches a kernel launch.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_address_and_ub_sanitizers(tmp_path):
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("another library is preloaded; the sanitizer runtime must come first")
    from linear_recurrent_attention_amd import build
    rt = build.sanitizer_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime beside the compiler")
    lib = build.build_sanitized()
    logs = str(tmp_path / "san")
    env = dict(os.environ,
               LD_PRELOAD=rt,
               ASAN_OPTIONS=f"detect_leaks=0:abort_on_error=1:log_path={logs}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={logs}",
               WKV_ABI_TEST_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = "".join(open(p).read() for p in sorted(glob.glob(logs + "*")))
    assert r.returncode == 0 and not reports, (
        f"exit {r.returncode}\n{reports[:4000]}\n{r.stdout[-3000:]}\n{r.stderr[-2000:]}")
    assert " passed" in r.stdout

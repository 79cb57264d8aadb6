"""The host code of libpa (argument checks, page-table validation, both planners, the
plan-matching and enqueue-side checks) under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds libpa.so with host-side -fsanitize=address,undefined (device code untouched) into
_build/sanitized/ and runs tests/test_host.py against it in a child process with the
sanitizer runtime preloaded (PA_LIBRARY names the library; leak checking is off because the
HIP runtime keeps allocations until exit).  Any sanitizer report fails the run."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


def _asan_runtime():
    if not os.path.exists(CLANG):
        return None
    path = subprocess.run([CLANG, "--print-file-name=libclang_rt.asan-x86_64.so"],
                          capture_output=True, text=True).stdout.strip()
    return path if os.path.isfile(path) else None


def test_host_tests_pass_under_address_and_undefined_behavior_sanitizers(tmp_path):
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("no clang AddressSanitizer runtime in this image")
    sys.path.insert(0, ROOT)
    from paged_attention_hd512_amd.build import build
    lib = build(sanitize=True)
    log = str(tmp_path / "sanitizer")
    env = dict(os.environ, LD_PRELOAD=runtime, PA_LIBRARY=lib,
               ASAN_OPTIONS=f"detect_leaks=0:abort_on_error=1:log_path={log}",
               UBSAN_OPTIONS=f"print_stacktrace=1:halt_on_error=1:log_path={log}")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_host.py"),
                        "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    reports = "".join(open(f).read() for f in glob.glob(log + "*"))
    assert not reports, reports[:4000]
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert " passed" in r.stdout

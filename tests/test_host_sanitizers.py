"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds libspecprefill.so with its host half instrumented (device code as
usual) and runs the C-ABI checks of test_abi.py against it in a child
process with the sanitizer runtime preloaded: argument checks, per-prompt
table builders, workspace layouts and window plans, on the CPU only. Any
report stops the child with a non-zero status.
"""
import os
import shutil
import subprocess
import sys

import pytest

from draft_attention_token_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc")
def test_abi_checks_clean_under_host_asan_and_ubsan(tmp_path):
    lib = build.build_sanitized(str(tmp_path))
    logs = tmp_path / "sanitizer"
    env = dict(os.environ)
    env.update({
        "SP_LIB_PATH": lib,
        "LD_PRELOAD": build.sanitizer_runtime(),
        # Python and torch are not instrumented: no leak report at exit, and
        # their own allocator pairings are not checked.
        "ASAN_OPTIONS": f"detect_leaks=0:alloc_dealloc_mismatch=0:halt_on_error=1:log_path={logs}",
        "UBSAN_OPTIONS": f"halt_on_error=1:print_stacktrace=1:log_path={logs}",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = ""
    for f in sorted(tmp_path.glob("sanitizer*")):
        reports += f.read_text()[:4000]
    assert r.returncode == 0 and not reports, (r.stdout[-2000:] + r.stderr[-2000:] + reports)

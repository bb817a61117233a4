"""The ABI tests again, against the host layer built with AddressSanitizer and
UndefinedBehaviorSanitizer (build.SANITIZE_OUT, built by build()).  Argument
validation never reaches the GPU, so the whole run needs none: the ABI tests
run in a child process with the clang ASan runtime preloaded and FA_LIBRARY
naming the sanitized library, and any sanitizer report fails it."""

import os
import subprocess
import sys

import pytest

from exact_attention_forward_fa_amd import build as fabuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_address_and_undefined_behavior_sanitizers(tmp_path):
    lib = fabuild.SANITIZE_OUT
    rt = fabuild.asan_runtime()
    if not os.path.exists(lib) or not rt:
        pytest.skip("sanitized host layer not built (run build()) or no ASan runtime")
    env = dict(os.environ, LD_PRELOAD=rt, FA_LIBRARY=lib,
               ASAN_OPTIONS=f"detect_leaks=0:abort_on_error=1:log_path={tmp_path}/asan",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={tmp_path}/ubsan")
    # the child really runs the sanitized build
    probe = subprocess.run([sys.executable, "-c",
                            "import ctypes, exact_attention_forward_fa_amd as fa; l = fa.load_library(); "
                            "print(l._name); ctypes.CDLL(None).__asan_init"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert probe.stdout.strip().endswith("libfa_sanitize.so")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", os.path.join(ROOT, "tests",
                        "test_abi.py")], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = [open(os.path.join(tmp_path, f)).read() for f in os.listdir(tmp_path)]
    assert not reports, "sanitizer reports:\n" + "\n".join(x[:3000] for x in reports)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout

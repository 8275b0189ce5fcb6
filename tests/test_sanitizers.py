"""The oracle and the C ABI's validation under AddressSanitizer and
UndefinedBehaviorSanitizer (host builds only, no GPU): the oracle's pins and
the ABI validation tests run against sanitized builds, with the sanitizer
runtimes preloaded into a separate Python process; any report fails."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.timeout(900)
def test_host_code_is_clean_under_sanitizers():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("the host compiler's sanitizer runtimes are not installed")
    env = dict(os.environ)
    pre = [asan, ubsan] + ([env["LD_PRELOAD"]] if env.get("LD_PRELOAD") else [])
    env["LD_PRELOAD"] = ":".join(pre)
    # the interpreter and torch keep memory until exit: leaks are not checked
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["OMP_NUM_THREADS"] = "4"
    r = subprocess.run([sys.executable, os.path.join(HERE, "sanitize", "run_host_checks.py")],
                       capture_output=True, text=True, env=env, timeout=880)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "[sanitizer run] oracle True, api True" in out, out[-2000:]

"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer (host only): every entry point over
small shapes (tests/oracle_sanitize_driver.c), with any report or leak failing the run. The oracle is the parity
reference, so a memory error in it would make its values, and every parity claim, meaningless."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sanitizer_build(out):
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fno-fast-math",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-pthread",
           os.path.join(ROOT, "oracle", "sdm_oracle.c"), os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"),
           "-lm", "-o", out]
    return subprocess.run(cmd, capture_output=True, text=True)


def test_oracle_clean_under_address_and_undefined_behaviour_sanitizers():
    if shutil.which("gcc") is None:
        pytest.skip("needs gcc")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "oracle_sanitize")
        b = _sanitizer_build(exe)
        if b.returncode != 0:
            if "asan" in b.stderr.lower() or "ubsan" in b.stderr.lower():
                pytest.skip("the sanitizer runtimes are not installed: " + b.stderr[-300:])
            raise AssertionError(b.stderr)
        # verify_asan_link_order=0: a library the environment preloads may come before the runtime
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:exitcode=23:verify_asan_link_order=0",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=24")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        report = r.stdout[-2000:] + r.stderr[-4000:]
        assert r.returncode == 0, report
        assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, report
        assert "all calls returned 0" in r.stdout, report

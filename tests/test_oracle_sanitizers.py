"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU):
every entry point on small seeded inputs (tests/oracle_sanitize_driver.c),
both norm scopes, both flush granularities, capacity overflow, a zero token,
the unquantized attention with n = 0.  Any out-of-bounds access, leak or
undefined operation fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "oracle"),
           os.path.join(ROOT, "oracle", "oscar_oracle.c"),
           os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"), "-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in r.stderr.lower() and "cannot find" in r.stderr.lower():
        pytest.skip("sanitizer runtime not installed")
    assert r.returncode == 0, r.stderr
    # a library preloaded by the environment may come before the sanitizer
    # runtime in the link order; that is allowed, not an error
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout, r.stderr[-3000:])

"""The CPU oracle under the host sanitizers.

Builds oracle/convrot_oracle.c together with tests/oracle_sanitize_main.c with
gcc's AddressSanitizer and UndefinedBehaviorSanitizer (no recovery: the first
report aborts) and runs it.  The driver calls every exported oracle function
on small, ragged and extreme inputs, so an out-of-bounds access, a use after
free, a signed overflow, a bad shift or an invalid float-to-integer
conversion anywhere in the oracle fails this test."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "oracle_sanitize")
        build = ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-Wno-unknown-pragmas",
                 "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                 os.path.join(HERE, "oracle_sanitize_main.c"), os.path.join(ROOT, "oracle", "convrot_oracle.c"),
                 "-o", exe, "-lm"]
        r = subprocess.run(build, capture_output=True, text=True)
        assert r.returncode == 0, "sanitizer build failed:\n" + r.stderr
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0 and "runtime error" not in r.stderr, (
            "sanitizer run failed (rc %d):\n%s\n%s" % (r.returncode, r.stdout, r.stderr[-4000:]))
        assert "oracle sanitizer run: ok" in r.stdout

"""The fp64 oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only): tests/oracle_sanitize.c runs every member's forward and
checkpointed backward on a tiny problem crossing the 64-token checkpoint,
checks the adjoints against central finite differences, and must exit cleanly
with no sanitizer report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    srcs = [os.path.join(ROOT, "tests", "oracle_sanitize.c"),
            os.path.join(ROOT, "oracle", "clr_oracle.c"), os.path.join(ROOT, "oracle", "conv_oracle.c")]
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", *srcs, "-o", exe, "-lm"]
    p = subprocess.run(cmd, capture_output=True, text=True)
    assert p.returncode == 0, p.stderr
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert "runtime error" not in r.stderr, r.stderr
    assert "AddressSanitizer" not in r.stderr, r.stderr
    assert r.returncode == 0, r.stderr
    assert "oracle sanitize: ok" in r.stdout

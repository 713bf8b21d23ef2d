"""The host C code (the oracle and the seeded input generator) built with AddressSanitizer
and UndefinedBehaviorSanitizer and run on a small workload with several threads: causal
and not, padded query rows, e4m3 and bf16 storage.  Any out-of-bounds access, leak or
undefined behaviour makes the sanitizer runtime fail the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_and_generator_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "sanitize_check")
    srcs = [os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "sa_synth", "synth.c"),
            os.path.join(ROOT, "oracle", "sanitize_check.c")]
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-o", exe] + srcs + ["-lm", "-lpthread"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("causal")]
    assert len(lines) == 3 and all(" rc 0 " in l for l in lines), r.stdout

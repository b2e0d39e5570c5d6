"""The fp64 oracle and the input generator (plain C, CPU only) built with
AddressSanitizer and UndefinedBehaviorSanitizer and run over every oracle
entry point by tests/sanitize/driver.c: any out-of-bounds access, leak,
use after free, signed overflow, misaligned or otherwise undefined operation
aborts the run.  (Host code only; the GPU library is not built here.)"""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_and_generator_under_asan_ubsan():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "driver")
        cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=all", "-o", exe, os.path.join(ROOT, "tests", "sanitize", "driver.c"),
               os.path.join(ROOT, "oracle", "moe_oracle.c"), os.path.join(ROOT, "synth", "moe_synth.c"),
               "-lm", "-lpthread"]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0, r.stdout + r.stderr
        assert r.stdout.startswith("checksum ")

"""The oracle's C code under gcc's AddressSanitizer and UndefinedBehaviorSanitizer.

oracle/sanitize_driver.c runs every oracle entry point (every fp16 pattern through the
conversions and the pair norm; score, K/V page quantization, unpacking, dequantization and
float64 decode over several configurations, including every packing width) on small seeded
inputs.  Built here with -fsanitize=address,undefined and no recovery, any out-of-bounds access,
leak or undefined operation ends the run with a non-zero status.  CPU only.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    odir = os.path.join(ROOT, "oracle")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer", "-I", odir,
                           os.path.join(odir, "pnmix_oracle.c"),
                           os.path.join(odir, "sanitize_driver.c"), "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "oracle sanitize driver: ok" in res.stdout

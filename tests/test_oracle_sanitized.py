"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize/oracle_driver.c calls every oracle function on random small
problems with exactly sized arrays; built with gcc and both sanitizers (host
code only), any out-of-bounds access, signed overflow or misaligned access in
the oracle aborts it.  CPU only."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_is_clean_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    build = subprocess.run(
        ["gcc", "-std=c99", "-O1", "-g", "-Wall", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
         os.path.join(HERE, "sanitize", "oracle_driver.c"), os.path.join(ROOT, "oracle", "ep_oracle.c"),
         "-lm", "-o", exe],
        capture_output=True, text=True)
    if build.returncode != 0 and "sanitizer" in (build.stderr + build.stdout).lower():
        pytest.skip("sanitizer runtime not available: " + build.stderr[-200:])
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "cases passed" in run.stdout

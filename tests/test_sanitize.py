"""The CPU oracle and the seeded input generators under AddressSanitizer and
UndefinedBehaviorSanitizer: tests/sanitize/driver.c calls every oracle entry
point and every generator on small inputs in exactly sized heap buffers, and
is built with oracle/oracle.c and synth/synth.c by gcc with
-fsanitize=address,undefined and no recovery, so any out-of-bounds access,
use after free, leak, signed overflow, bad shift or misaligned load ends the
run with a report. The same command runs by hand:

  gcc -O1 -g -std=c11 -fsanitize=address,undefined -fno-sanitize-recover=all \\
      -fno-omit-frame-pointer -ffp-contract=off -fopenmp \\
      tests/sanitize/driver.c oracle/oracle.c synth/synth.c -lm -o /tmp/qmv_sanitize && /tmp/qmv_sanitize

gcc -flto -Wlto-type-mismatch over the same three files checks that the
driver's declarations match the definitions.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [os.path.join(ROOT, p) for p in ("tests/sanitize/driver.c", "oracle/oracle.c", "synth/synth.c")]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_and_generators_run_clean_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "qmv_sanitize"
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-ffp-contract=off", "-fopenmp"] + SOURCES + ["-lm", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="4")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "run clean" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_driver_declarations_match_the_definitions(tmp_path):
    cmd = ["gcc", "-O1", "-flto", "-Wlto-type-mismatch", "-Werror", "-std=c11", "-fopenmp", "-ffp-contract=off"]
    r = subprocess.run(cmd + SOURCES + ["-lm", "-o", str(tmp_path / "lto_check")], capture_output=True, text=True,
                       cwd=str(tmp_path))
    assert r.returncode == 0, r.stderr[-4000:]

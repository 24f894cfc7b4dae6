"""The streaming C oracle under AddressSanitizer and UndefinedBehaviorSanitizer
(host code only): its driver (``oracle/kpa_oracle_check.c``) runs the oracle
over a fixed set of shapes; the sanitized build must report nothing and print
exactly what the plain build prints."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "oracle", "kpa_oracle.c"), os.path.join(ROOT, "oracle", "kpa_oracle_check.c")]


def _build(out, flags):
    subprocess.check_call(["gcc", "-std=c11", "-Wall", "-Wno-unknown-pragmas", *flags, "-o", out, *SRC, "-lm"])


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    san = str(tmp_path / "oracle_san")
    plain = str(tmp_path / "oracle_plain")
    _build(san, ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                 "-fno-sanitize-recover=all"])
    _build(plain, ["-O2"])
    # verify_asan_link_order=0: the process may have other libraries preloaded
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r_san = subprocess.run([san], capture_output=True, text=True, env=env, timeout=300)
    assert r_san.returncode == 0, r_san.stderr[-4000:]
    assert "runtime error" not in r_san.stderr and "AddressSanitizer" not in r_san.stderr, r_san.stderr[-4000:]
    r_plain = subprocess.run([plain], capture_output=True, text=True, timeout=300)
    assert r_plain.returncode == 0, r_plain.stderr
    assert r_san.stdout == r_plain.stdout
    assert r_plain.stdout.count("case ") == 7

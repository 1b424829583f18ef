"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/native/oracle_sanitized.c compiles the oracle's C source into one
program with gcc's -fsanitize=address,undefined (no recovery) and drives
every entry point over small batches full of edge cases (NaN and +inf
logits, greedy and infinite temperatures, p, top-k and min-p at their
limits, bf16 and strided rows, per-row keys, out-of-range history ids, bad
arguments).  Any out-of-bounds access, leak, use after free, overflow or
misaligned access makes it abort.  CPU only."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "native", "oracle_sanitized.c")


def _build_and_run(tmp_path, *defines):
    exe = str(tmp_path / ("oracle_sanitized" + "".join(defines)))
    build = ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Werror=incompatible-pointer-types",
             *defines, "-o", exe, DRIVER, "-lm"]
    r = subprocess.run(build, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    r = _build_and_run(tmp_path)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_the_sanitizer_catches_a_planted_overrun(tmp_path):
    r = _build_and_run(tmp_path, "-DPLANT_OVERRUN")
    # (UBSan's object-size check or ASan's redzone, whichever sees it first)
    caught = "heap-buffer-overflow" in r.stderr or "insufficient space for an object" in r.stderr
    assert r.returncode != 0 and caught, r.stdout + r.stderr[-2000:]

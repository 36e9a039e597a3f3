"""The CPU oracle under sanitizers (CPU only).

* AddressSanitizer + UndefinedBehaviorSanitizer: oracle/sanitize_driver.c
  calls every oracle entry point on small seeded inputs and edge cases
  (ragged vocabularies, K = vocab, a budget of 0, empty contexts, commits at
  the end of their region, mask rows of several words).
* UndefinedBehaviorSanitizer: the oracle's pin tests, run in a child process
  against a UBSan build of the same source.
"""
import os
import subprocess
import sys

import pytest

from oracle import build as ob

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _can_sanitize(tmp_path, flags):
    src = tmp_path / "probe.c"
    src.write_text("int main(void) { return 0; }\n")
    r = subprocess.run(["gcc", *flags, "-o", str(tmp_path / "probe"), str(src)],
                       capture_output=True, text=True)
    return r.returncode == 0


def test_driver_under_asan_and_ubsan(tmp_path):
    if not _can_sanitize(tmp_path, ob.ASAN_UBSAN):
        pytest.skip("gcc here has no address/undefined sanitizer runtime")
    exe = ob.build_sanitize_driver(str(tmp_path))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", OMP_NUM_THREADS="2")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "sanitize driver ok" in r.stdout


def test_pins_under_ubsan(tmp_path):
    if not _can_sanitize(tmp_path, ob.UBSAN):
        pytest.skip("gcc here has no undefined-behaviour sanitizer runtime")
    lib = ob.build(ubsan=True)
    pins = ["tests/test_oracle_topk.py", "tests/test_oracle_tree.py",
            "tests/test_oracle_mask_attn.py", "tests/test_oracle_accept.py",
            "tests/test_oracle_commit.py", "tests/test_oracle_selective.py",
            "tests/test_oracle_layer.py"]
    env = dict(os.environ, TD_ORACLE_LIB=lib, UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="4")
    # the child loads the sanitized build ...
    who = subprocess.run([sys.executable, "-c", "import oracle; print(oracle._load()._name)"],
                         cwd=ROOT, capture_output=True, text=True, env=env, timeout=120)
    assert who.returncode == 0 and who.stdout.strip() == lib, who.stdout + who.stderr
    # ... and runs every pin against it
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", *pins],
                       cwd=ROOT, capture_output=True, text=True, env=env, timeout=900)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout and "failed" not in r.stdout

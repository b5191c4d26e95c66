"""The oracle's pins under AddressSanitizer and UndefinedBehaviorSanitizer.

The C oracle is rebuilt with -fsanitize=address,undefined (host code only)
and the oracle pin suites run against it in a child process that preloads
the ASan runtime.  Any out-of-bounds access, use after free or undefined
behaviour in the oracle (or in the seeded input generator's calls into it)
aborts the child.  CPU only.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_oracle_pins.py", "tests/test_oracle_gqa.py", "tests/test_oracle_calib.py",
          "tests/test_oracle_curve.py", "tests/test_oracle_shared.py"]


def _asan_runtime():
    try:
        path = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_pass_under_asan_and_ubsan():
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    env = dict(os.environ)
    # the ASan runtime must come first; anything already preloaded stays
    pre = os.environ.get("LD_PRELOAD", "").strip()
    env.update(TRI_ORACLE_SANITIZE="1", LD_PRELOAD=asan + (" " + pre if pre else ""),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu"] + SUITES, cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out

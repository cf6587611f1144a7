"""The oracle's pins, re-run against an AddressSanitizer +
UndefinedBehaviorSanitizer build of the oracle (a separate shared library
built from the same source; any report aborts the run).  The two exhaustive
2^32-pattern encoder sweeps are left out here (they run in the normal suite
and would take minutes under the sanitizers)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PINS = ["tests/test_oracle_codecs.py", "tests/test_oracle_quant.py", "tests/test_oracle_gemm.py",
        "tests/test_oracle_dequant.py", "tests/test_oracle_kv.py", "tests/test_oracle_combine.py",
        "tests/test_oracle_delayed.py", "tests/test_oracle_pack.py"]


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from oracle import build
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = build.build_sanitized(str(tmp_path / "liboracle_san.so"))
    env = dict(os.environ)
    env.update(FP8_ORACLE_LIB=lib, LD_PRELOAD=asan, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", "-k", "not exhaustive_brute_force"] + PINS,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out

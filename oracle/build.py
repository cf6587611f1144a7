"""Build the CPU oracle (TEST INFRASTRUCTURE ONLY) with gcc.

The oracle is plain C11, compiled at -O2 with no fast-math and no
floating-point contraction so that every fp32 operation is one IEEE binary32
operation rounded to nearest even.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libfp8_oracle.so")
SRC = os.path.join(HERE, "fp8_oracle.c")


FLAGS = ["-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"]
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build_sanitized(out: str, verbose: bool = False) -> str:
    """The same oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
    (any report aborts), for running the oracle's pins under them; load it
    with libasan preloaded and FP8_ORACLE_LIB pointing at `out`."""
    cmd = ["gcc", "-O1"] + FLAGS + SANITIZE + ["-o", out, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    return out


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2"] + FLAGS + ["-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)

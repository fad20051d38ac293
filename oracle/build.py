"""Compile the C oracle (test infrastructure; see ``oracle/__init__.py``).

Plain gcc, -O2, no fast-math, OpenMP over independent chains.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")
# GDN_ORACLE_LIBRARY names another build (the sanitized one of the CPU tests)
LIB = os.environ.get("GDN_ORACLE_LIBRARY") or os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build_sanitized(out: str, cc: str = "/opt/rocm/llvm/bin/clang") -> str:
    """The oracle with AddressSanitizer and UndefinedBehaviorSanitizer (clang,
    so that one sanitizer runtime serves it and the HIP library's host code)."""
    cmd = [cc, "-O1", "-g", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-o", out, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(verbose=True))

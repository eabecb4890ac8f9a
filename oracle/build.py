"""Builds the oracle's shared library with gcc (test infrastructure only).

The oracle is plain C with no GPU code; it is compiled here, next to its
source, so that tests and the bench's CPU-baseline leg can load it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "topk_oracle.c")
SOURCES = [SOURCE, os.path.join(HERE, "sample_oracle.c")]
LIBRARY = os.path.join(HERE, "liboracle_topk.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-D_POSIX_C_SOURCE=200809L", "-Wall", "-Wextra",
           "-fPIC", "-shared", "-pthread", "-o", LIBRARY + ".tmp"] + SOURCES + ["-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIBRARY + ".tmp", LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))

"""Build the CPU reference library ``oracle/libmxoracle.so`` with gcc.

Test infrastructure: the oracle is built so the test suite, the smoke check and
the benchmark's CPU-baseline leg can load it. No product code links it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmxoracle.so")


def build(verbose: bool = False) -> str:
    """Compile mx_oracle.c; returns the path of the shared library."""
    cmd = [
        "gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fopenmp", "-fPIC", "-shared",
        os.path.join(HERE, "mx_oracle.c"), "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

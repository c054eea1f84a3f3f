"""Build the reference oracle (test infrastructure) with gcc.

fp64 loops in written order: -ffp-contract=off keeps every a*b+c as two
roundings, exactly as the source reads.  OpenMP only parallelises over
independent outputs (rows, samples, requests), never inside a sum.
"""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose=False):
    src = os.path.join(_HERE, "oracle.c")
    out = os.path.join(_HERE, "liboracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter", src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose=True)

"""Build liboracle.so (host only: gcc, OpenMP, no HIP).

The oracle is test infrastructure; building it is not using it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
# ISO C with no contraction and no fast-math: every binary32 operation of the
# quantizer rounds exactly once, as written.
CFLAGS = ["-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-ffp-contract=off", "-fno-fast-math"]


def build(src: str = None, out: str = None, verbose: bool = False) -> str:
    src = src or os.path.join(HERE, "oracle.c")
    out = out or os.path.join(HERE, "liboracle.so")
    cmd = ["gcc", *CFLAGS, src, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))

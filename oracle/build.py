"""Builds the oracle's shared library with the host C compiler (test infrastructure)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build() -> str:
    src = os.path.join(HERE, "agmm_oracle.c")
    out = os.path.join(HERE, "liboracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", "-std=c11",
           src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())

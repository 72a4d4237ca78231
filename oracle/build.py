"""Build the C oracle (test infrastructure) into oracle/libkda_oracle.so.

Plain gcc, -O2, OpenMP over (sequence, head) pairs; no fast-math, so every
floating-point operation is the IEEE fp64 one written in kda_oracle.c.
"""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def build(src=None, out=None, extra_flags=()):
    src = src or os.path.join(_HERE, "kda_oracle.c")
    out = out or os.path.join(_HERE, "libkda_oracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", *extra_flags,
           src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())

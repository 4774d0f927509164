"""Compile the seeded input generator into synth/libsynth.so."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libsynth.so")
SRC = [os.path.join(HERE, "synth.c")]


def build(force=True):
    if not force and os.path.exists(LIB) and all(os.path.getmtime(LIB) >= os.path.getmtime(s) for s in SRC):
        return LIB
    # -O2: at -O3 gcc vectorizes around the libm calls and runs several times
    # slower here.  -ffp-contract=off keeps every float operation separately rounded, so the
    # bytes do not depend on the compiler's choice of fused multiply-adds.
    cmd = ["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-mavx2", "-Wall", "-Wextra", "-o", LIB + ".tmp"] + SRC + ["-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build())

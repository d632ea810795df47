"""Build the CPU oracle (test infrastructure): gcc, -O2, no fast-math, no FMA."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "librro.so")
SRC = os.path.join(HERE, "rro.c")


def build_oracle(force: bool = True) -> str:
    """Compile oracle/rro.c into oracle/librro.so and return the path."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
           "-fPIC", "-shared", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_oracle())

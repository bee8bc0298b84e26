"""Build the CPU oracle shared libraries (test infrastructure only).

liboracle_f32.so : float arithmetic (the precision the model file fixes)
liboracle_f64.so : the same source in double, used to bound the float build's drift

Flags: -O3 -ffp-contract=off and no fast-math, so products are rounded before
they are added and no sum is reassociated.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gpt2_oracle.c")
FLAGS = ["-O3", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11", "-Wall"]


def lib_path(kind: str) -> str:
    return os.path.join(HERE, f"liboracle_{kind}.so")


def build(verbose: bool = False) -> None:
    for kind, extra in (("f32", []), ("f64", ["-DORACLE_REAL_IS_DOUBLE"])):
        out = lib_path(kind)
        cmd = ["gcc", *FLAGS, *extra, "-o", out + ".tmp", SRC, "-lm"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

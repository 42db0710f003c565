"""Builds the f64 oracle shared library with gcc (plain -O2, no fast-math)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "ssm_oracle.c"), os.path.join(HERE, "conv_oracle.c")]
LIB_PATH = os.path.join(HERE, "libssm_oracle.so")


def build_oracle(verbose=False):
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", *SRCS, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH

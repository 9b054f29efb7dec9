"""Builds the CPU oracle library (oracle/liboracle.so) with gcc.

Test infrastructure only: the library is the checker, not the product.
Compiled without fast-math so the k loop is summed exactly as written.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ref_gemm.c")              # GEMM, codecs, activations
SRC_ATTENTION = os.path.join(HERE, "ref_attention.c")   # softmax, attention
SRC_LAYERNORM = os.path.join(HERE, "ref_layernorm.c")   # residual + LayerNorm linear
SRC_CONV = os.path.join(HERE, "ref_conv.c")             # 2-D convolution
SOURCES = [SRC, SRC_ATTENTION, SRC_LAYERNORM, SRC_CONV]
LIB = os.path.join(HERE, "liboracle.so")
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11", "-Wall", "-Wextra",
          "-shared", "-fPIC", "-pthread"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, *SOURCES, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Build oracle/liboracle.so with gcc (test infrastructure only)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
OUT = os.path.join(HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-adds beyond the explicit fmaf calls, so
# every fp32 operation is the single IEEE-rounded one the source states.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra"]


def build(extra=(), out=OUT, src=SRC):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1:]))

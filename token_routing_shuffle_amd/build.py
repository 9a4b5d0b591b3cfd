"""Build libmoe.so (HIP, gfx950) and its device-data-check variant
libmoe_debug.so in-tree with hipcc.

    python -m token_routing_shuffle_amd.build
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoe.so")
SOURCES = ["api.hip", "route.hip", "shuffle.hip", "ffn.hip", "combine.hip", "srs_sag.hip", "cosched.hip", "noalloc.hip"]
HEADERS = ["common.h", "internal.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed fp32 instructions (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


VARIANTS = {
    # release: the product library
    "release": (LIB, []),
    # device data checks: kernels also record clamped input values in the
    # workspace error word (moe_debug_errors)
    "debug": (os.path.join(HERE, "libmoe_debug.so"), ["-DMOE_DEBUG_CHECKS=1"]),
}


def build_variant(name, verbose=False):
    out, defines = VARIANTS[name]
    bdir = os.path.join(BUILD, name)
    os.makedirs(bdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(bdir, src + ".o")
        cmd = [HIPCC, *FLAGS, *defines, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
        if verbose:
            print(" ".join(cmd))
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, out)
    return out


def build(verbose=False):
    """Both libraries; returns the release library's path."""
    with ThreadPoolExecutor(max_workers=2) as ex:
        paths = list(ex.map(lambda n: build_variant(n, verbose), ["release", "debug"]))
    return paths[0]


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

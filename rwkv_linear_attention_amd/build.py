"""Ahead-of-time build of libwkv7.so for gfx950 with hipcc (no JIT).

The library is built in-tree next to this file so that it travels with the
source tree; nothing is installed into site-packages.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libwkv7.so")
SOURCES = ["wkv7_api.hip", "wkv7_recurrent.hip", "wkv7_step.hip", "wkv7_chunked.hip", "wkv7_chunked_f32.hip", "wkv7_backward.hip",
           "wkv7_gdn_bwd.hip", "wkv7_noalloc.hip"]
HEADERS = ["wkv7_common.hpp", "wkv7_internal.hpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # Keep packed-fp32 VALU instructions out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def inputs():
    return sources() + [os.path.join(CSRC, h) for h in HEADERS] + [os.path.join(ROOT, "include", "wkv7.h")]


def is_stale():
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in inputs())


def build(force=True, verbose=False):
    """Compile every HIP source into libwkv7.so (always, when force)."""
    if not force and not is_stale():
        return LIB
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc] + HIPCC_FLAGS + ["-I" + os.path.join(ROOT, "include")] + sources() + ["-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd, stderr=subprocess.STDOUT if verbose else subprocess.DEVNULL)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose=True))

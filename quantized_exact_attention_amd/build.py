"""Builds the gfx950 HIP library in-tree: _lib/libsage_mi355x.so.

hipcc, gfx950 only, -O3, no FMA contraction unless written explicitly (the
prepass must reproduce plain FP32 arithmetic bit for bit), and packed FP32
instructions disabled.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_lib")
LIB = os.path.join(OUT_DIR, "libsage_mi355x.so")
SOURCES = ["prep_kernels.hip", "attn_mainloop.hip", "sage_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"),
]


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile the library; returns its path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    if not force and os.path.exists(LIB):
        newest = max(os.path.getmtime(p) for p in srcs + [os.path.join(CSRC, h) for h in
                                                            ("sage_device.hpp", "sage_launch.hpp")])
        if os.path.getmtime(LIB) >= newest:
            return LIB
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; harmless
    noise = "is not a recognized feature for this target"
    errs = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, errs))
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

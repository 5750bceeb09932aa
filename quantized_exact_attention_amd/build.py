"""Builds the gfx950 HIP library in-tree: _lib/libsage_mi355x.so.

hipcc, gfx950 only, -O3, no FMA contraction unless written explicitly (the
prepass must reproduce plain FP32 arithmetic bit for bit), and packed FP32
instructions disabled.

The build also checks the compiler's resource report of every kernel and
fails when a kernel uses scratch memory (register spills), or when the
mainloop kernel needs more than 168 VGPRs or falls below three waves per
SIMD.  The mainloop's design rests on both: three independent workgroups per
CU (each wave at most 512/3 registers), and a tile-load pipeline whose waits
count exactly the tile loads in flight, which a scratch access (also a
vector-memory operation) would silently break.
"""
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_lib")
LIB = os.path.join(OUT_DIR, "libsage_mi355x.so")
SOURCES = ["prep_kernels.hip", "attn_mainloop.hip", "sage_noalloc.hip", "issue_probe.hip", "sage_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# What the mainloop kernel may use: registers for three waves per SIMD.
MAINLOOP_KERNEL = "mainloop_kernel"
MAINLOOP_MAX_VGPRS = 168
MAINLOOP_MIN_OCCUPANCY = 3

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"),
    "-Rpass-analysis=kernel-resource-usage",
]


def kernel_resources(text: str) -> dict:
    """Per-kernel resource figures from the compiler's kernel-resource-usage
    remarks: {mangled name: {"VGPRs": n, "AGPRs": n, "ScratchSize": n,
    "Occupancy": n, "VGPRs Spill": n, ...}}."""
    out = {}
    cur = None
    for line in text.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^]]*\])?: (\d+) \[-Rpass-analysis", line)
        if m and cur is not None:
            cur[m.group(1)] = int(m.group(2))
    return out


def check_resources(res: dict) -> list:
    """Problems with the kernels' resources (empty when all is well)."""
    problems = []
    if not any(MAINLOOP_KERNEL in k for k in res):
        problems.append("no resource report for %s" % MAINLOOP_KERNEL)
    for name, r in res.items():
        if r.get("ScratchSize", 0) != 0 or r.get("VGPRs Spill", 0) != 0:
            problems.append("%s uses scratch memory (%d bytes per lane, %d VGPRs spilled)"
                            % (name, r.get("ScratchSize", 0), r.get("VGPRs Spill", 0)))
        if MAINLOOP_KERNEL in name:
            regs = r.get("VGPRs", 0) + r.get("AGPRs", 0)
            if regs > MAINLOOP_MAX_VGPRS:
                problems.append("%s needs %d VGPRs + AGPRs, more than %d (three waves per SIMD)"
                                % (name, regs, MAINLOOP_MAX_VGPRS))
            if r.get("Occupancy", 0) < MAINLOOP_MIN_OCCUPANCY:
                problems.append("%s runs %d waves per SIMD, fewer than %d"
                                % (name, r.get("Occupancy", 0), MAINLOOP_MIN_OCCUPANCY))
    return problems


def _noise(line: str) -> bool:
    # the host pass does not know the packed-fp32 feature and says so;
    # resource remarks are parsed, not shown
    return "is not a recognized feature for this target" in line or "remark:" in line or \
        re.match(r"^\s*(\d+\s*)?\|", line) is not None


def build(force: bool = True, verbose: bool = False, csrc: str = CSRC, out: str = None) -> str:
    """Compile the library (sources from `csrc`, output `out`, by default the
    in-tree library); returns its path.  Raises when hipcc fails or the
    kernels' resources break the limits above."""
    lib = out or LIB
    srcs = [os.path.join(csrc, s) for s in SOURCES]
    if not force and os.path.exists(lib):
        newest = max(os.path.getmtime(p) for p in srcs + [os.path.join(csrc, h) for h in
                                                            ("sage_device.hpp", "sage_launch.hpp")])
        if os.path.getmtime(lib) >= newest:
            return lib
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    stderr = res.stderr or ""
    errs = "\n".join(l for l in stderr.splitlines() if not _noise(l))
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, errs))
    problems = check_resources(kernel_resources(stderr))
    if problems:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("kernel resources out of bounds:\n  " + "\n  ".join(problems))
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))

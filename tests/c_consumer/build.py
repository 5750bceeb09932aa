"""Builds the plain-C consumer of the library's C ABI (a test program):
tests/c_consumer/_build/sage_c_consumer, linked against the in-tree
libsage_mi355x.so and the HIP runtime."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "sage_c_consumer.c")
OUT = os.path.join(HERE, "_build", "sage_c_consumer")
LIB_DIR = os.path.join(ROOT, "quantized_exact_attention_amd", "_lib")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(force: bool = True) -> str:
    if not force and os.path.exists(OUT) and os.path.getmtime(OUT) >= os.path.getmtime(SRC):
        return OUT
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROCM, "include"), SRC, "-o", OUT,
           "-L" + LIB_DIR, "-lsage_mi355x", "-Wl,-rpath,$ORIGIN/../../../quantized_exact_attention_amd/_lib",
           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("gcc failed (%d):\n%s" % (res.returncode, res.stderr))
    return OUT


if __name__ == "__main__":
    print(build())

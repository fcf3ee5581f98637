"""Build helper for the plain C consumer of the C ABI (tests/c/ra_c_consumer.c)."""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "blockwise_ring_attention_amd")
SRC = os.path.join(HERE, "c", "ra_c_consumer.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out_path: str) -> str:
    """gcc, C11, against include/ra.h and the in-tree libra.so; the rpath finds both
    libraries at run time."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include"), SRC, "-L", PKG, "-lra", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-lm", f"-Wl,-rpath,{PKG}:{os.path.join(ROCM, 'lib')}", "-o", out_path]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed:\n{r.stdout}\n{r.stderr}")
    return out_path

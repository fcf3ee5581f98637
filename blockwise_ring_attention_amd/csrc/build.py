"""Build libra.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc.

Usage: python -m blockwise_ring_attention_amd.csrc.build  [--jobs N] [--ablations]
Always recompiles; the library lands next to the package's __init__.py. With
--ablations (or build_ablations()) it also builds one comparison library per
design-choice switch of ra_fwd.hip / ra_host.cpp into the package's ablation/ folder:
the same entry points and results, computed without that choice, for measurement only;
and the diagnostic build (per-workgroup timeline of the bf16 kernel) beside them.
"""

from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libra.so")
ABLATION_DIR = os.path.join(PKG, "ablation")
SOURCES = ["ra_host.cpp", "ra_fwd.hip", "ra_merge.hip"]
# name -> preprocessor switch (see the top of ra_fwd.hip)
ABLATIONS = {
    "xcd_scatter": "RA_ABLATION_XCD_SCATTER",
    "no_swizzle": "RA_ABLATION_NO_SWIZZLE",
    "no_skip": "RA_ABLATION_NO_SKIP",
    "one_head": "RA_ABLATION_ONE_HEAD",
    "stage_barrier": "RA_ABLATION_STAGE_BARRIER",
}
# Diagnostic builds, made beside the ablations: the same results, plus recording.
DIAGNOSTICS = {
    "timeline": "RA_DIAG_TIMELINE",   # per-workgroup clock stamps, HW_ID and XCC_ID (ra_diag_timeline)
}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed-fp32 VALU forms are kept out of every kernel. Inputs are taken to be NaN-free,
# which lets max reductions skip canonicalising moves.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-fno-honor-nans"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include"), "-I", HERE]


def _compile(src: str, build_dir: str, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    # A fixed compilation-unit ID per source: hipcc otherwise derives it from the source's
    # path and writes it into symbol names, so the same sources built in another
    # directory would give a library with other bytes.
    cuid = "ra_" + os.path.splitext(src)[0]
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, f"-cuid={cuid}", *[f"-D{d}" for d in defines], "-c",
           os.path.join(HERE, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", *DEVICE_FLAGS, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(jobs: int = 3, verbose: bool = False) -> str:
    build_dir = os.path.join(ROOT, "_build")
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir), SOURCES))
    _link(objs, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def ablation_path(name: str) -> str:
    return os.path.join(ABLATION_DIR, f"libra_{name}.so")


def build_ablations(jobs: int = 3, verbose: bool = False) -> list[str]:
    """One library per design-choice switch (same C ABI), for A/B measurement, and one
    per diagnostic switch."""
    os.makedirs(ABLATION_DIR, exist_ok=True)
    out = []

    def one(item):
        name, define = item
        bdir = os.path.join(ROOT, "_build", f"ablation_{name}")
        os.makedirs(bdir, exist_ok=True)
        objs = [_compile(s, bdir, (define,)) for s in SOURCES]
        _link(objs, ablation_path(name))
        return ablation_path(name)

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        out = list(ex.map(one, [*ABLATIONS.items(), *DIAGNOSTICS.items()]))
    if verbose:
        for p in out:
            print(f"built {p}")
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=3)
    ap.add_argument("--ablations", action="store_true", help="also build the design-choice comparison libraries")
    args = ap.parse_args()
    build(args.jobs, verbose=True)
    if args.ablations:
        build_ablations(args.jobs, verbose=True)
    sys.exit(0)

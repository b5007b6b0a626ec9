"""Build libh3block.so (HIP sources for gfx950) in-tree.

    python -m video_diffusion_transformer_dit_amd.build [--jobs N] [--verbose]

Each source is compiled to an object under _build/ in parallel, then linked
into video_diffusion_transformer_dit_amd/libh3block.so. The build always
recompiles (it is the "does it build" check as well as the build)."""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libh3block.so")

SOURCES = ["validate.cpp", "runtime.hip", "elementwise.hip", "gemm.hip", "attention.hip", "attention_fixed.hip",
           "sparse.hip", "gemm_mxfp8.hip", "mx_quant.hip", "block.hip", "ceiling.hip"]
# Per-source device flags. attention_fixed.hip selects the VGPR form of the
# MFMA instructions (accumulators in VGPRs unless a register-class hint says
# otherwise), so its score accumulators need no copy out of AGPRs.
EXTRA = {"attention_fixed.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-fPIC", "-std=c++17", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
# Packed FP32 (v_pk_*_f32) instructions are disabled for all device code.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, verbose: bool) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC] + COMMON + ["-c", path, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = DEVICE + EXTRA.get(src, [])
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{msg}")
    if msg.strip() and verbose:
        print(msg)
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    jobs = jobs or min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)), 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libh3block.so failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--clean", action="store_true")
    a = ap.parse_args(argv)
    if a.clean and os.path.isdir(BUILD):
        shutil.rmtree(BUILD)
    print(build(a.jobs, a.verbose))
    return 0


if __name__ == "__main__":
    sys.exit(main())

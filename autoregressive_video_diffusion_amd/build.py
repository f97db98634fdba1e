"""Build libcrattn.so (HIP for gfx950) in-tree with hipcc.

    python -m autoregressive_video_diffusion_amd.build [--jobs N]

The assembly of the dense attention's key loop is generated first
(csrc/gen_attn_loop.py -> csrc/attn_loop.inc).  Each source is compiled to an
object in parallel, then linked into
``autoregressive_video_diffusion_amd/libcrattn.so``.  Packed-fp32 VALU
instructions are disabled for all device code.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
OUT = os.path.join(HERE, "libcrattn.so")
ARCH = "gfx950"
SOURCES = ["api.cpp", "plan.cpp", "rope.hip", "attn.hip", "qkv.hip", "hsa.hip", "svg2.hip"]
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return p


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc(), "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
           "-Wall", "-Wno-unused-function", "-c", os.path.join(CSRC, src), "-o", obj,
           *DEVICE_FLAGS]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    msgs = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if any(msgs):
        print("\n".join(msgs))
    return obj


def generate() -> None:
    """Regenerate the assembly of the attention key loop (attn_loop.inc)."""
    subprocess.run([sys.executable, os.path.join(CSRC, "gen_attn_loop.py"), "--out",
                    os.path.join(CSRC, "attn_loop.inc")], check=True)


def build(jobs: int | None = None) -> str:
    generate()
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    args = ap.parse_args()
    print(build(args.jobs))

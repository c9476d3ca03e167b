"""Build libmla.so for gfx950 with hipcc (in-tree, next to this file).

    python -m head_latent_attention_14_amd.build [--jobs N] [--save-temps DIR]
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
LIB = os.path.join(HERE, "libmla.so")
SOURCES = ["api.cpp", "append.hip", "decode_attn.hip", "decode_attn_stream.hip", "decode_attn_h32.hip",
           "decode_gemm.hip", "prefill.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 VALU instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]
# MFMA accumulators in ordinary VGPRs: the softmax rescale and the partial
# stores then touch them without AGPR<->VGPR copies every tile. Not for the
# 128-head kernel, whose value accumulators fill the accumulation registers.
PER_SOURCE = {src: ["-mllvm", "-amdgpu-mfma-vgpr-form=1"] for src in SOURCES
              if src not in ("api.cpp", "decode_attn_h32.hip")}


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *lang, *COMMON, *PER_SOURCE.get(src, []), *extra, "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l
                     and "warning: unknown target feature" not in l)
    if warn.strip():
        sys.stderr.write(warn + "\n")
    return obj


def build(jobs: int = 4, save_temps: str | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    extra = []
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        extra = [f"-save-temps={'obj'}"]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--save-temps", default=None)
    a = ap.parse_args()
    print(build(a.jobs, a.save_temps))


if __name__ == "__main__":
    main()

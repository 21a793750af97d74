"""Build libdspark.so (HIP C++ for gfx950) in-tree.

    python -m draft_verify_sampling_bias_amd.build [--jobs N] [--save-temps DIR]

Every source under csrc/ is compiled with hipcc for --offload-arch=gfx950 and
linked into draft_verify_sampling_bias_amd/libdspark.so.  Packed-fp32 VALU
instructions are disabled for all device code.
"""
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
OUT = os.path.join(PKG, "libdspark.so")
BUILD_DIR = os.path.join(PKG, "_build")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]

# bias_tile.hip: MFMA results in architectural registers (the 64-row kernel
# keeps its W2 fragments in all 256 accumulation registers; with accumulation-
# register results the compiler moves some fragments out and back and reads
# every result through v_accvgpr_read)
PER_SOURCE = {"bias_tile.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

SOURCES = ["plan.cpp", "api.hip", "bias_tile.hip", "finish.hip", "verify.hip", "schedule.hip", "pack.hip", "capacity.hip",
           "calibrate.hip", "check.hip", "noalloc.hip", "rnn.hip"]


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    per = PER_SOURCE.get(src, [])
    cmd = [HIPCC, *COMMON, *per, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and per and "Unknown command line argument" in r.stderr:
        # a compiler without that backend option: the same code, a few
        # instructions per chunk slower
        sys.stderr.write(f"[{src}] {' '.join(per)} not known to this compiler; building without it\n")
        cmd = [HIPCC, *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write(f"[{src}]\n" + "\n".join(noise) + "\n")
    return obj


def build(jobs: int = 8, save_temps: str | None = None, verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = []
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        extra = [f"-save-temps={'obj'}", "-Rpass-analysis=kernel-resource-usage"]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("--save-temps", default=None)
    args = ap.parse_args()
    build(args.jobs, args.save_temps)


if __name__ == "__main__":
    main()

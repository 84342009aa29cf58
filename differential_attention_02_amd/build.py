"""Build libdiffattn.so (HIP kernels for gfx950 + the C ABI) in-tree.

Usage: python -m differential_attention_02_amd.build [--resource-usage]

Each source under csrc/ is compiled by hipcc to an object in _build/ (in
parallel), then linked into differential_attention_02_amd/libdiffattn.so.
Packed fp32 instructions are disabled for all device code.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdiffattn.so")
ARCH = "gfx950"

COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument"]


# Per-source code-generation options.  fwd_onepass.hip: two waves per SIMD,
# all 256 registers ordinary VGPRs (the default form put the score products in
# accumulation registers and copied them back).  The other kernels were
# measured and are faster without it.
EXTRA = {"fwd_onepass.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, resource_usage: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if resource_usage and src.endswith(".hip"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if resource_usage:
        lines = [ln for ln in r.stderr.splitlines() if "remark" in ln or "Function Name" in ln]
        if lines:
            print("\n".join(lines))
    return obj


def build(resource_usage: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "api.cpp")]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, resource_usage), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--resource-usage", action="store_true", help="print per-kernel register/LDS use")
    args = ap.parse_args(argv)
    print(build(args.resource_usage))
    return 0


if __name__ == "__main__":
    sys.exit(main())

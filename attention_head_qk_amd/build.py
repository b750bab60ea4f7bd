"""Build libgqa.so (the gfx950 HIP kernels and the C ABI of include/gqa.h) in-tree.

Usage: python attention_head_qk_amd/build.py [--verbose] [--resource-usage]

(Run as a file, not as a package module: importing the package loads libgqa.so, which must
not be required in order to rebuild it.)

Every HIP source is compiled with hipcc for gfx950 only, with packed-fp32 instruction
selection switched off (-Xclang -target-feature -Xclang -packed-fp32-ops), then linked into
attention_head_qk_amd/libgqa.so next to this file.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgqa.so")
ARCH = "gfx950"

SOURCES = ["gqa_api.hip", "prologue.hip", "prefill_bf16.hip", "prefill_f32.hip", "decode.hip"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libgqa)")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{INCLUDE}", f"-I{CSRC}"]


def _compile(src: str, verbose: bool, resource_usage: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    if resource_usage:
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, resource_usage), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.verbose or a.resource_usage, a.resource_usage))


if __name__ == "__main__":
    sys.exit(main())

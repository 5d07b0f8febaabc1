"""Build libfa.so for gfx950 in-tree with hipcc.

Usage: python -m attention_fa_fwd_06_amd.build [--verbose] [--resource-usage]

Each translation unit compiles in its own process (the three kernel files
hold one element type each), then one link step makes
attention_fa_fwd_06_amd/libfa.so.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"

SOURCES = ["fa_api.cpp", "fa_kernels_f32.hip", "fa_kernels_f16.hip", "fa_kernels_bf16.hip"]

COMMON = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are kept out of the generated code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libfa.so")


def _compile(src: str, resource_usage: bool, build_dir: str, defines: list[str]) -> tuple[str, str]:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src), "-o", obj]
    if resource_usage and src.endswith(".hip"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def build(verbose: bool = False, resource_usage: bool = False, defines=(), out: str = LIB,
          build_dir: str = BUILD) -> str:
    """Compile every source and link `out` (default: the in-tree libfa.so).

    defines: extra preprocessor definitions, e.g. tile overrides for sweeps.
    """
    defines = list(defines)
    os.makedirs(build_dir, exist_ok=True)
    jobs = min(len(SOURCES), os.cpu_count() or 1)
    logs = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_compile, s, resource_usage, build_dir, defines) for s in SOURCES]
        objs = []
        for f in futs:
            obj, log = f.result()
            objs.append(obj)
            logs.append(log)
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose or resource_usage:
        for log in logs:
            lines = [ln for ln in log.splitlines() if "packed-fp32-ops" not in ln]
            if lines:
                print("\n".join(lines))
        print(f"built {out}")
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true")
    ap.add_argument("-D", dest="defines", action="append", default=[], help="extra preprocessor definition")
    ap.add_argument("--out", default=LIB, help="output library path")
    ap.add_argument("--build-dir", default=BUILD)
    args = ap.parse_args(argv)
    build(verbose=args.verbose, resource_usage=args.resource_usage, defines=args.defines, out=args.out,
          build_dir=args.build_dir)


if __name__ == "__main__":
    sys.exit(main())

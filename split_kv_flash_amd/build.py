"""Ahead-of-time build of the HIP library ``libsplitkv.so`` for gfx950.

Compiles every source under ``csrc/`` with hipcc into ``_build/`` at the
repository root and links the shared library next to this file, where the
Python binding loads it. Run ``python -m split_kv_flash_amd.build``.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from typing import List, Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libsplitkv.so"
ARCH = "gfx950"

SOURCES = ["api.hip", "gqa_split.hip", "combine.hip", "mla_split.hip", "project.hip", "query_tile.hip", "read_probe.hip"]

# -packed-fp32-ops: keep the compiler from emitting packed FP32 arithmetic; the
# host pass warns that it does not know the feature, which is harmless.
BASE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; a ROCm toolchain is required to build libsplitkv.so")


def build(out_dir: Optional[str] = None, defines: Sequence[str] = (), jobs: int = 8,
          resource_report: bool = False, build_dir: Optional[str] = None,
          quiet: bool = True) -> str:
    """Compile and link; returns the library path. Always recompiles."""
    out_dir = out_dir or PKG
    build_dir = build_dir or os.path.join(ROOT, "_build")
    os.makedirs(build_dir, exist_ok=True)
    cc = hipcc()
    extra: List[str] = [f"-D{d}" for d in defines]
    if resource_report:
        extra.append("-Rpass-analysis=kernel-resource-usage")

    def compile_one(src: str) -> str:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *BASE_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        log = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{log}")
        if log.strip() and (not quiet or resource_report):
            print(log, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    lib = os.path.join(out_dir, LIB_NAME)
    tmp = lib + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)
    return lib


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("-D", dest="defines", action="append", default=[], help="extra -D define")
    ap.add_argument("--out-dir", default=None)
    ap.add_argument("--build-dir", default=None)
    ap.add_argument("--resource-report", action="store_true",
                    help="print per-kernel VGPR/AGPR/LDS/occupancy from the compiler")
    ap.add_argument("-j", "--jobs", type=int, default=8)
    args = ap.parse_args(argv)
    lib = build(args.out_dir, args.defines, args.jobs, args.resource_report, args.build_dir,
                quiet=False)
    print(lib)


if __name__ == "__main__":
    main()

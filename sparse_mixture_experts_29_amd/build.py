"""Build libmoe.so (gfx950) in-tree: one hipcc compile per source, then a shared link.

    python -m sparse_mixture_experts_29_amd.build [--jobs N] [--out PATH] [-D NAME=VALUE ...]

Every source is compiled every time (the build check must compile, not reuse). --out and -D
build a variant of the same sources elsewhere (tuning macros such as MOE_GEMM_*), which the
binding loads when MOE_LIB names it; the in-tree library is unchanged by such a build.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmoe.so")
BUILD = os.path.join(ROOT, "_build")
SOURCES = ["api.hip", "router.hip", "permute.hip", "grouped_mlp.hip", "grouped_mlp_small.hip", "combine.hip",
           "backward.hip", "pack.hip", "grouped_mlp_wide.hip", "grouped_mlp_decode.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
    # no packed fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature name: harmless, filtered
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{err}")
    return err


def build(jobs: int = 8, verbose: bool = False, out: str = OUT, defines=()) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    # a variant build keeps its objects apart from the in-tree ones
    bdir = BUILD if out == OUT else os.path.join(BUILD, "variant_" + os.path.basename(out).replace(".", "_"))
    os.makedirs(bdir, exist_ok=True)
    objs = []
    dflags = [f"-D{d}" for d in defines]

    def compile_one(src):
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        msg = _run([HIPCC, *CFLAGS, *dflags, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and msg:
            print(msg, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, out)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--out", default=OUT, help="where to write the library (default: in-tree)")
    ap.add_argument("-D", dest="defines", action="append", default=[], help="extra preprocessor define NAME=VALUE")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose, os.path.abspath(a.out), a.defines))


if __name__ == "__main__":
    main()

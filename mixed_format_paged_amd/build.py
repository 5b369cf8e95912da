"""Build libmkv.so (the HIP library behind include/mkv.h) for gfx950, in-tree.

Usage: python -m mixed_format_paged_amd.build [--jobs N]
Each csrc/*.hip file is compiled to an object under _build/ in parallel, then
linked into mixed_format_paged_amd/libmkv.so.  Always recompiles.
"""
import argparse
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmkv.so")
BUILD = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep fp32 arithmetic in unpacked VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    return src, obj, r.returncode, err


def build(jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or min(8, len(srcs))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, srcs))
    bad = [r for r in results if r[2] != 0]
    # every compiler diagnostic of the HIP sources is shown, not only on failure
    for src, _, rc, err in results:
        if err.strip():
            print(f"== {os.path.basename(src)}\n{err}", file=sys.stderr)
    if bad:
        raise RuntimeError("HIP compile failed: " + ", ".join(os.path.basename(b[0]) for b in bad))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [r[1] for r in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    a = ap.parse_args()
    print(build(a.jobs))

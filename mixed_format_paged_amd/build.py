"""Build libmkv.so (the HIP library behind include/mkv.h) for gfx950, in-tree.

Usage: python -m mixed_format_paged_amd.build [--jobs N] [--item-trace]
Each csrc/*.hip file is compiled to an object under _build/ in parallel, then
linked into mixed_format_paged_amd/libmkv.so.  Always recompiles.
--item-trace builds the measurement variant instead (MKV_ITEM_TRACE=1: the
attention kernels record per-workgroup timestamps, read back with
mkv_debug_item_trace) into mixed_format_paged_amd/libmkv_trace.so.
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
TRACE_OUT = os.path.join(PKG, "libmkv_trace.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep fp32 arithmetic in unpacked VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _compile(src, build_dir=BUILD, extra=()):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    return src, obj, r.returncode, err


def build(jobs=None, item_trace=False):
    build_dir = os.path.join(BUILD, "trace") if item_trace else BUILD
    out = TRACE_OUT if item_trace else OUT
    extra = ("-DMKV_ITEM_TRACE=1",) if item_trace else ()
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or min(8, len(srcs))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda src: _compile(src, build_dir, extra), srcs))
    bad = [r for r in results if r[2] != 0]
    # every compiler diagnostic of the HIP sources is shown, not only on failure
    for src, _, rc, err in results:
        if err.strip():
            print(f"== {os.path.basename(src)}\n{err}", file=sys.stderr)
    if bad:
        raise RuntimeError("HIP compile failed: " + ", ".join(os.path.basename(b[0]) for b in bad))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [r[1] for r in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--item-trace", action="store_true", help="build the item-trace variant (libmkv_trace.so)")
    a = ap.parse_args()
    print(build(a.jobs, a.item_trace))

"""Host code of the library under AddressSanitizer and UndefinedBehaviorSanitizer,
on the CPU.

The library is built again into a temporary directory with the sanitizers on
its host code only (`-Xarch_host`; the device code is compiled as usual and
never runs here), and the C-ABI tests (tests/test_abi.py: every declared
symbol, shape and range checks, every host validation error, workspace
sizing) run against that build in a child Python process, with the sanitizer
runtime preloaded (Python itself is not instrumented) and any report fatal.
"""
import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SANITIZE = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _asan_runtime():
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/lib/llvm/bin/clang"
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_under_host_sanitizers(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("sanitizer runtime not found")
    srcs = sorted(glob.glob(os.path.join(ROOT, "mixed_format_paged_amd", "csrc", "*.hip")))
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17", "-I", os.path.join(ROOT, "include"),
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument"]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, *flags, *SANITIZE, "-c", src, "-o", obj], capture_output=True, text=True)
        return src, obj, r

    with ThreadPoolExecutor(max_workers=8) as ex:
        results = list(ex.map(compile_one, srcs))
    for src, _, r in results:
        assert r.returncode == 0, f"{src}:\n{r.stderr[-3000:]}"
    lib = str(tmp_path / "libmkv_sanitized.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libasan", *SANITIZE[:2],
                        "-o", lib, *[o for _, o, _ in results]], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, LD_PRELOAD=rt, MKV_LIB_PATH=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert "passed" in r.stdout

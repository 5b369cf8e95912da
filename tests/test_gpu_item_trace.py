"""The item-trace build (MKV_ITEM_TRACE=1, libmkv_trace.so) records a sane
per-workgroup timeline and changes no result: the same decode through the
product library and through the trace library gives the same bytes.  Each
library runs in its own child process (the binding loads one library per
process)."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PRODUCT = os.path.join(ROOT, "mixed_format_paged_amd", "libmkv.so")
TRACE = os.path.join(ROOT, "mixed_format_paged_amd", "libmkv_trace.so")

CHILD = r"""
import math, sys
import numpy as np
sys.path.insert(0, sys.argv[1])
import torch
import mixed_format_paged_amd as M
import workloads as W
from workloads.device_cache import DeviceWorkload
w = W.scaled(W.WORKLOADS["ragged-32x4096-65536"], B=3, L=1, lengths=("list", (2000, 700, 3100)), recent_tokens=64)
st = W.make_structure(w)
dw = DeviceWorkload(w, st, "cuda")
layout = (w.Hq, w.Hkv, w.d)
ws = torch.empty(M.mkv_decode_workspace_bytes(layout, w.B, dw.bt.numel(), 1), dtype=torch.uint8, device="cuda")
out = torch.full((w.B, w.Hq, w.d), float("nan"), device="cuda")
lse = torch.full((w.B, w.Hq), float("nan"), device="cuda")
M.mkv_decode_attn(layout, dw.cache.pools[0], dw.batch(), dw.q[0].contiguous(), 1 / math.sqrt(w.d), out, lse, ws)
assert M.mkv_workspace_status(ws) == 0
np.save(sys.argv[2], np.concatenate([out.cpu().numpy().ravel(), lse.cpu().numpy().ravel()]))
if sys.argv[3] == "trace":
    buf = np.zeros((4096, 32), dtype=np.uint64)
    M.mkv_debug_item_trace(buf)
    np.save(sys.argv[4], buf)
print("child done", flush=True)
"""


def _run(lib, out, trace=None):
    env = dict(os.environ, MKV_LIB_PATH=lib)
    args = [sys.executable, "-c", CHILD, ROOT, out, "trace" if trace else "plain", trace or ""]
    r = subprocess.run(args, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]


@pytest.mark.gpu
@pytest.mark.skipif(not os.path.exists(TRACE), reason="trace build missing (python -m mixed_format_paged_amd.build --item-trace)")
def test_item_trace_build_records_a_timeline_and_changes_no_result(tmp_path):
    a, b, tr = str(tmp_path / "a.npy"), str(tmp_path / "b.npy"), str(tmp_path / "t.npy")
    _run(PRODUCT, a)
    _run(TRACE, b, tr)
    assert np.array_equal(np.load(a), np.load(b), equal_nan=True)
    t = np.load(tr).astype(np.int64)
    used = (t[:, 3] & 0xFFFFFFFF) > 0
    assert used.sum() > 0
    t = t[used]
    # entry <= fragments built <= partial stored, on the constant clock
    assert np.all(t[:, 0] > 0) and np.all(t[:, 0] <= t[:, 1]) and np.all(t[:, 1] <= t[:, 2])
    first, lend = t[:, 4:16], t[:, 16:28]
    has = first > 0
    assert has.any()
    # a wave's first page lands after entry, its loop ends after that, and before the store
    assert np.all(first[has] >= np.repeat(t[:, [0]], 12, axis=1)[has])
    assert np.all(lend[has] >= first[has])
    assert np.all(lend[has] <= np.repeat(t[:, [2]], 12, axis=1)[has])
    # the item words name valid requests and KV heads
    assert np.all(((t[:, 3] >> 48) & 0xFFFF) < 3) and np.all(((t[:, 3] >> 40) & 0xFF) < 4)

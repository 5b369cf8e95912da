#!/usr/bin/env python3
"""Mixed FP8 / TQ3 paged decode attention on one MI355X: the canary workload.

Workload (default): 2 requests x 59,008 tokens, 16 attention layers with one
cache each, 24 query / 4 KV heads, head_dim 256, pages of 16 tokens; the last
1,024 tokens and the first 8 pages of each request are FP8, the other 3,616
pages per request TQ3; physical pages shuffled (the pages' direct-decode
canary shape, arXiv 2608.23834, page 1, Abstract).  Inputs are synthetic and
seeded (workloads/), generated on the GPU, resident in HBM before timing.

One step = one decode step of the whole path, layers in sequence as a model
runs them:
    plan (block tables + tier map -> per-format page lists and split-K chunks)
    for each of the 16 layers:
        append the step's new token (K, V of both requests, FP8 E4M3), inside
        the partial-attention launch (mkv_append_attend)
        FP8 and TQ3 partial kernels (one launch), log-sum-exp merge
    demote, in all 16 layers, the page of each request that leaves the recent
    window (FP8 -> TQ3 pack, written to a spare TQ3 slot so the cache state
    stays identical from step to step)
The step is captured once in a HIP graph and replayed.

Prints one JSON line.  `value` is KV GB/s: algorithmic KV bytes of the 16
layers (every page of every request read once per layer) / step time.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="canary-2x59008-16L")
    ap.add_argument("--kernel", choices=["mfma", "valu"], default="mfma")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--separate-append", action="store_true",
                    help="append with its own launch (mkv_append) instead of inside the attend launch")
    ap.add_argument("--no-control", action="store_true", help="skip the same-run all-FP8 control")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the CPU oracle")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workloads")
    ap.add_argument("--cpu-units", type=int, default=6, help="(layer, request, KV head) units the oracle is timed on")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 5 times (counter calibration)")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="only run this many eager steps (for rocprofv3), print nothing else")
    ap.add_argument("--pack-only", type=int, default=0, metavar="REPS",
                    help="only time the pack of 8,192 random pages (REPS launches back to back) and print it")
    ap.add_argument("--item-trace", type=int, default=0, metavar="REPS",
                    help="only trace REPS partial-attention launches with the item-trace build "
                         "(mixed_format_paged_amd/libmkv_trace.so) and print their per-workgroup timeline")
    return ap.parse_args()


class Runner:
    """Holds the device state of one workload and enqueues its decode steps."""

    def __init__(self, w, st, all_fp8=False, kernel="mfma", fused_append=True):
        import torch
        import mixed_format_paged_amd as M
        from workloads.device_cache import DeviceWorkload
        import workloads as W
        self.M, self.torch = M, torch
        if all_fp8:
            # the control: identical shapes with every page FP8 (no demotion at build)
            import numpy as np
            st = W.Structure(st.seq_lens, st.n_pages, st.bt_offsets,
                             np.where(st.tiers == W.TIER_S, W.TIER_R, st.tiers).astype(np.uint8),
                             st.staging_ids, st.staging_ids, st.n_fp8, 0,
                             np.zeros(0, dtype=np.int64), np.zeros(0, dtype=np.int64))
        self.w, self.st = w, st
        self.fused_append = fused_append and kernel == "mfma"
        M.set_partial_kind(1 if kernel == "mfma" else 0)
        t0 = time.time()
        self.dw = DeviceWorkload(w, st, "cuda", spare_tq3=w.B)
        torch.cuda.synchronize()
        self.build_s = time.time() - t0
        self.layout = (w.Hq, w.Hkv, w.d)
        self.batch = self.dw.batch()
        self.sm_scale = 1.0 / math.sqrt(w.d)
        dev = "cuda"
        L, B = w.L, w.B
        self.ws = torch.empty(M.mkv_decode_workspace_bytes(self.layout, B, self.dw.bt.numel(), 1),
                              dtype=torch.uint8, device=dev)
        self.out = torch.empty((L, B, w.Hq, w.d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((L, B, w.Hq), dtype=torch.float32, device=dev)
        g = torch.Generator(device=dev)
        g.manual_seed(12345)
        self.k_new = torch.randn((L, B, 1, w.Hkv, w.d), generator=g, device=dev)
        self.v_new = torch.randn((L, B, 1, w.Hkv, w.d), generator=g, device=dev)
        self.pos = (self.dw.seq_lens - 1).clamp(min=0).contiguous()
        # the page leaving the recent window: logical page n - recent_pages of each request
        rec = w.recent_tokens // 16
        ent = [int(st.bt_offsets[b]) + max(0, int(st.n_pages[b]) - rec) for b in range(B)]
        self.dem_src = self.dw.bt[torch.as_tensor(ent, device=dev)].contiguous()
        is_fp8 = bool((self.dem_src < st.n_fp8).all())
        self.dem_src = self.dem_src if is_fp8 else torch.zeros(0, dtype=torch.int32, device=dev)
        n_tq3_total = self.dw.cache.n_tq3
        self.dem_dst = torch.arange(n_tq3_total - B, n_tq3_total, dtype=torch.int32, device=dev) + st.n_fp8
        self.dem_dst = self.dem_dst[:self.dem_src.numel()].contiguous()
        self.q = [self.dw.q[l].contiguous() for l in range(L)]

    def step(self):
        M, dw, lay, bat, ws = self.M, self.dw, self.layout, self.batch, self.ws
        M.mkv_decode_plan(lay, dw.cache.pools[0], bat, 1, ws)
        for l in range(self.w.L):
            if self.fused_append:
                M.mkv_append_attend(lay, [dw.cache.pools[l]], bat, self.k_new[l], self.v_new[l], self.q[l],
                                    self.sm_scale, self.out[l], self.lse[l], ws)
            else:
                M.mkv_append(lay, dw.cache.pools[l], self.k_new[l], self.v_new[l], dw.bt_offsets, dw.bt, self.pos)
                M.mkv_attend(lay, [dw.cache.pools[l]], bat, self.q[l], self.sm_scale, self.out[l], self.lse[l], ws)
        if self.dem_src.numel():
            M.mkv_demote_pages_layers(lay, dw.cache.pools, self.dem_src, self.dem_dst)

    def kv_bytes(self):
        """Algorithmic KV bytes per step: every page of every request, every layer."""
        import numpy as np
        st, w = self.st, self.w
        fb = self.M.mkv_fp8_page_bytes(self.layout)
        tb = self.M.mkv_tq3_page_bytes(self.layout)
        n_t = int((st.tiers == 2).sum())
        n_f = int(st.total_pages - n_t)
        return w.L * (n_f * fb + n_t * tb), w.L * n_t * tb, n_t * tb

    def time_steps(self, steps, warmup, graph=True):
        torch = self.torch
        run = self.step
        if graph:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                for _ in range(2):
                    self.step()
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            self.graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(self.graph):
                self.step()
            run = self.graph.replay
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        # an event between consecutive steps: the mean is first to last, and
        # each step's own time gives the spread
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        evs[0].record()
        for i in range(steps):
            run()
            evs[i + 1].record()
        torch.cuda.synchronize()
        per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
        self.step_p10 = per[int(0.1 * (steps - 1))]
        self.step_median = per[(steps - 1) // 2]
        self.step_p90 = per[int(0.9 * (steps - 1))]
        return evs[0].elapsed_time(evs[-1]) / steps

    def time_kernels(self, reps=32):
        """Average and median duration of the partial-attention launch (both
        formats, one layer) and of the merge launch, with HIP events recorded
        on the stream the kernels are launched on.  Launch i reads layer
        i mod L, so, as in the step, no launch finds its layer's pages in the
        last-level cache from the launch before."""
        torch, M = self.torch, self.M
        lay, bat, ws, L = self.layout, self.batch, self.ws, self.w.L
        M.mkv_decode_plan(lay, self.dw.cache.pools[0], bat, 1, ws)
        part = lambda l: M.mkv_attend_partials(lay, [self.dw.cache.pools[l]], bat, self.q[l], self.sm_scale, ws)
        merge = lambda l: M.mkv_merge(lay, 1, bat, self.out[l], self.lse[l], ws)
        res = {}
        for name in ("partials", "merge"):
            for l in range(min(L, 3)):
                part(l)
                merge(l)
            torch.cuda.synchronize()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for i, (a, b) in enumerate(evs):
                l = i % L
                if name == "merge":
                    part(l)
                a.record()
                part(l) if name == "partials" else merge(l)
                b.record()
            torch.cuda.synchronize()
            ms = sorted(a.elapsed_time(b) for a, b in evs)
            res[name] = (sum(ms) / len(ms), ms[len(ms) // 2])
        return res


def item_trace(runner, reps):
    """Per-workgroup timeline of the partial-attention launch, from the
    item-trace build (mkv_debug_item_trace: the 100 MHz constant clock at
    points of each workgroup's item).  Each repetition runs partials + merge
    on two layers back to back, then partials on a third, and reads the trace
    of that last launch.  Returns a dict of percentiles (p10, p50, p90, max)
    in microseconds, pooled over the repetitions."""
    import numpy as np
    torch, M = runner.torch, runner.M
    lay, bat, ws, L = runner.layout, runner.batch, runner.ws, runner.w.L
    M.mkv_decode_plan(lay, runner.dw.cache.pools[0], bat, 1, ws)
    part = lambda l: M.mkv_attend_partials(lay, [runner.dw.cache.pools[l]], bat, runner.q[l], runner.sm_scale, ws)
    merge = lambda l: M.mkv_merge(lay, 1, bat, runner.out[l], runner.lse[l], ws)
    keys = ("entry", "fragments_built", "first_page_landed", "page_loop", "loop_end_spread_in_wg",
            "last_loop_end_to_stored", "stored", "stored_tq3_items", "stored_fp8_items")
    acc = {k: [] for k in keys}
    buf = np.zeros((4096, 32), dtype=np.uint64)
    items = None
    for i in range(reps + 1):
        l0 = (3 * i) % L
        part(l0)
        merge(l0)
        part((l0 + 1) % L)
        merge((l0 + 1) % L)
        part((l0 + 2) % L)
        torch.cuda.synchronize()
        M.mkv_debug_item_trace(buf)
        if i == 0:
            continue                                    # warm-up
        info = buf[:, 3].astype(np.int64)
        used = (info & 0xFFFFFFFF) > 0
        t = buf[used].astype(np.int64)
        items = int(used.sum())
        us = lambda x: (x - t[:, 0].min()) / 100.0     # 100 MHz clock -> us from the first entry
        first, lend = t[:, 4:16], t[:, 16:28]
        valid = first > 0
        acc["entry"] += list(us(t[:, 0]))
        acc["fragments_built"] += list((t[:, 1] - t[:, 0]) / 100.0)
        acc["first_page_landed"] += list(((first - t[:, [0]]) / 100.0)[valid])
        acc["page_loop"] += list(((lend - first) / 100.0)[valid])
        for wg in range(t.shape[0]):
            v = valid[wg]
            if v.any():
                acc["loop_end_spread_in_wg"].append((lend[wg][v].max() - lend[wg][v].min()) / 100.0)
                acc["last_loop_end_to_stored"].append((t[wg, 2] - lend[wg][v].max()) / 100.0)
        acc["stored"] += list(us(t[:, 2]))
        tq3 = ((t[:, 3] >> 32) & 0xFF) == 1
        acc["stored_tq3_items"] += list(us(t[tq3, 2]))
        acc["stored_fp8_items"] += list(us(t[~tq3, 2]))
    pct = lambda v: [round(float(x), 2) for x in np.percentile(np.array(v), [10, 50, 90, 100])] if v else None
    return {"workgroups": items, "reps": reps, **{k: pct(v) for k, v in acc.items()}}


def time_materialize(runner, reps=8):
    """The dense shadow the decode path avoids: dequantise every page of every
    request of one layer to BF16 K and V (mkv_materialize, one launch per
    request), timed with HIP events on the launching stream; launch set i reads
    layer i mod L.  Returns (avg ms, bytes read, bytes written) per layer."""
    torch, M = runner.torch, runner.M
    w, st = runner.w, runner.st
    n_pages = [int(x) for x in st.n_pages]
    shape = (max(n_pages) * 16, w.Hkv, w.d)
    K = torch.empty(shape, dtype=torch.int16, device="cuda")
    V = torch.empty(shape, dtype=torch.int16, device="cuda")

    def run(l):
        for b in range(w.B):
            M.mkv_materialize(runner.layout, runner.dw.cache.pools[l], runner.batch, b, 0, n_pages[b], K, V)

    run(0)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        run(i % w.L)
        b.record()
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in evs) / reps
    read = runner.kv_bytes()[0] // w.L
    written = sum(n_pages) * 16 * w.Hkv * w.d * 2 * 2
    del K, V
    return ms, read, written


def time_multi_query(runner, T=4, reps=8):
    """mkv_decode_attn_multi (plan + partials + merge) on one layer of the
    canary with each request's last T tokens as causal queries, timed with HIP
    events; launch set i reads layer i mod L.  Returns (avg ms per layer)."""
    torch, M = runner.torch, runner.M
    w = runner.w
    g = torch.Generator(device="cuda")
    g.manual_seed(17)
    q = torch.randn((1, w.B, T, w.Hq, w.d), generator=g, device="cuda")
    out = torch.empty((1, w.B, T, w.Hq, w.d), device="cuda")
    lse = torch.empty((1, w.B, T, w.Hq), device="cuda")
    ws = torch.empty(M.mkv_decode_workspace_bytes_multi(runner.layout, w.B, runner.dw.bt.numel(), 1, T),
                     dtype=torch.uint8, device="cuda")

    def run(l):
        M.mkv_decode_attn_multi(runner.layout, [runner.dw.cache.pools[l]], runner.batch, q, runner.sm_scale, out, lse, ws)

    run(0)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        run(i % w.L)
        b.record()
    torch.cuda.synchronize()
    if M.mkv_workspace_status(ws) != 0:
        raise RuntimeError("multi-query decode status")
    return sum(a.elapsed_time(b) for a, b in evs) / reps


def time_demote_pack(runner, n_pages=8192, reps=10, scales=(1.0, 1.0)):
    """The pack kernel at the 64 requests x 128 aging pages scale: n_pages FP8
    pages of random E4M3 bytes (no NaN codes) demoted into n_pages TQ3 slots,
    one layer (mkv_demote_pages) with layer scales (k_scale, v_scale), timed
    with HIP events.  Returns (avg ms, bytes read + written)."""
    torch, M = runner.torch, runner.M
    lay = runner.layout
    fb, tb = M.mkv_fp8_page_bytes(lay), M.mkv_tq3_page_bytes(lay)
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    fp8 = torch.randint(0, 254, (n_pages, fb), dtype=torch.uint8, generator=g, device="cuda")
    fp8 += (fp8 >= 0x7F).to(torch.uint8)              # skip the NaN codes 0x7F and 0xFF
    tq3 = torch.empty((n_pages, tb), dtype=torch.uint8, device="cuda")
    tier = torch.full((2 * n_pages,), M.TIER_FREE, dtype=torch.uint8, device="cuda")
    pool = M.make_pool(fp8, tq3, tier, n_pages, n_pages, k_scale=scales[0], v_scale=scales[1])
    src = torch.arange(n_pages, dtype=torch.int32, device="cuda")
    dst = src + n_pages
    M.mkv_demote_pages(lay, pool, src, dst)
    torch.cuda.synchronize()
    # back-to-back launches between one pair of events: the average launch
    # duration, as the kernel trace reports it (plus the launch gaps)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        M.mkv_demote_pages(lay, pool, src, dst)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del fp8, tq3
    return ms, n_pages * (fb + tb)


def time_lifecycle(runner, reps=8):
    """mkv_lifecycle_step at a page boundary of the canary (every request starts
    a page and ages one Recent page into TQ3 in all layers), on block-table rows
    with one spare entry; the tables, tier map and free stacks are restored
    between repetitions (not timed).  Returns (avg ms, pages demoted)."""
    torch, M = runner.torch, runner.M
    w, st, dw = runner.w, runner.st, runner.dw
    dev = "cuda"
    n_fp8, n_tq3 = dw.cache.n_fp8, dw.cache.n_tq3
    n_pages = [int(x) for x in st.n_pages]
    offs = [0]
    for n in n_pages:
        offs.append(offs[-1] + n + 1)
    bt0 = torch.full((offs[-1],), -1, dtype=torch.int32, device=dev)
    for b in range(w.B):
        bt0[offs[b]:offs[b] + n_pages[b]] = dw.bt[int(st.bt_offsets[b]):int(st.bt_offsets[b + 1])]
    seq0 = torch.tensor([16 * n for n in n_pages], dtype=torch.int32, device=dev)
    tier = dw.cache.tier
    tier0 = tier.clone()
    free_f = torch.nonzero(tier[:n_fp8] == M.TIER_FREE).flatten().to(torch.int32)
    free_t = (torch.nonzero(tier[n_fp8:] == M.TIER_FREE).flatten() + n_fp8).to(torch.int32)
    ff0 = torch.zeros(n_fp8, dtype=torch.int32, device=dev)
    tf0 = torch.zeros(n_tq3, dtype=torch.int32, device=dev)
    ff0[:free_f.numel()] = free_f
    tf0[:free_t.numel()] = free_t
    tops0 = torch.tensor([free_f.numel(), free_t.numel()], dtype=torch.int32, device=dev)
    offs_d = torch.tensor(offs, dtype=torch.int32, device=dev)
    bt, seq, ff, tf, tops = bt0.clone(), seq0.clone(), ff0.clone(), tf0.clone(), tops0.clone()
    ws = torch.zeros(M.mkv_lifecycle_workspace_bytes(w.B), dtype=torch.uint8, device=dev)
    R = w.recent_tokens // 16
    ms = []
    for _ in range(reps):
        for x, x0 in ((bt, bt0), (seq, seq0), (tier, tier0), (ff, ff0), (tf, tf0), (tops, tops0)):
            x.copy_(x0)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        M.mkv_lifecycle_step(runner.layout, dw.cache.pools, offs_d, bt, seq, tier, ff, tf, tops, R, ws)
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    status = M.mkv_workspace_status(ws)
    demoted = int(tops0[1] - tops[1])
    tier.copy_(tier0)
    torch.cuda.synchronize()
    if status != 0:
        raise RuntimeError(f"lifecycle step status {status}")
    return sum(ms[1:]) / (reps - 1), demoted


def time_rotated(runner, reps=16):
    """Rotated TQ3 pages: layer 0 of the workload built again with a sign
    vector (its TQ3 pages rotated), and the attention of one layer (plan, the
    query rotation, partials with the back-rotation, merge: mkv_attend after
    mkv_decode_plan) timed against the same call on the plain layer 0, with HIP
    events, alternating; plus mkv_demote_pages of 8,192 random E4M3 pages with
    the rotation.  Returns a dict of ms."""
    import numpy as np
    torch, M = runner.torch, runner.M
    import workloads as W
    from workloads.device_cache import DeviceWorkload
    w, st = runner.w, runner.st
    signs = np.where(np.random.default_rng(5).integers(0, 2, w.d) == 0, 1, -1).astype(np.int8)
    dwr = DeviceWorkload(w, st, "cuda", layers=[0], tq3_signs=[signs])
    lay, bat = runner.layout, runner.batch
    ws = torch.empty(M.mkv_decode_workspace_bytes(lay, w.B, runner.dw.bt.numel(), 1), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.B, w.Hq, w.d), device="cuda")
    lse = torch.empty((w.B, w.Hq), device="cuda")
    q = runner.q[0]
    M.mkv_decode_plan(lay, runner.dw.cache.pools[0], bat, 1, ws)

    def run(pool):
        M.mkv_attend(lay, [pool], bat, q, runner.sm_scale, out, lse, ws)

    for pool in (dwr.cache.pools[0], runner.dw.cache.pools[0]):
        run(pool)
    torch.cuda.synchronize()
    res = {"rot": [], "plain": []}
    for i in range(2 * reps):
        pool, key = (dwr.cache.pools[0], "rot") if i % 2 == 0 else (runner.dw.cache.pools[0], "plain")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run(pool)
        b.record()
        torch.cuda.synchronize()
        res[key].append(a.elapsed_time(b))
    status = M.mkv_workspace_status(ws)
    # the rotated pack
    n_pages = 8192
    fb, tb = M.mkv_fp8_page_bytes(lay), M.mkv_tq3_page_bytes(lay)
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    fp8 = torch.randint(0, 254, (n_pages, fb), dtype=torch.uint8, generator=g, device="cuda")
    fp8 += (fp8 >= 0x7F).to(torch.uint8)
    tq3 = torch.empty((n_pages, tb), dtype=torch.uint8, device="cuda")
    tier = torch.full((2 * n_pages,), M.TIER_FREE, dtype=torch.uint8, device="cuda")
    sg = torch.as_tensor(signs, device="cuda")
    pool = M.make_pool(fp8, tq3, tier, n_pages, n_pages, tq3_signs=sg)
    src = torch.arange(n_pages, dtype=torch.int32, device="cuda")
    dst = src + n_pages
    M.mkv_demote_pages(lay, pool, src, dst)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(5):
        M.mkv_demote_pages(lay, pool, src, dst)
    b.record()
    torch.cuda.synchronize()
    dem = a.elapsed_time(b) / 5
    del dwr, fp8, tq3
    torch.cuda.empty_cache()
    if status != 0:
        raise RuntimeError(f"rotated attend status {status}")
    rot, plain = sum(res["rot"]) / reps, sum(res["plain"]) / reps
    return {"attend_merge_ms_per_layer": round(rot, 5), "plain_attend_merge_ms_per_layer": round(plain, 5),
            "vs_plain": round(rot / plain, 3), "demote_8192_pages_ms": round(dem, 5),
            "demote_gbs": round(n_pages * (fb + tb) / (dem * 1e-3) / 1e9, 2)}


def kernel_source_hash():
    """Hash of the sources the partial-attention kernel is compiled from."""
    import hashlib
    h = hashlib.sha256()
    for f in ("mkv_partial_mfma.hip", "mkv_internal.h", "mkv_format.h"):
        with open(os.path.join(ROOT, "mixed_format_paged_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload):
    """HBM bytes per partial-attention launch from the committed counter
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_attend_{workload}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return int(float(rec["hbm_bytes_per_launch"]))


def copy_calibration(nbytes, reps):
    """A plain device-to-device copy of known size, for scaling the FETCH_SIZE /
    WRITE_SIZE counters to bytes."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[bench] copy calibration: {reps} copies of {nbytes} bytes", file=sys.stderr, flush=True)


def oracle_units(w, st, picks, out, new_kv=None):
    """The CPU oracle on sampled (layer, request, KV head) units: its value
    path (quantise -> dequantise) and fp64 dense attention for the unit's G
    query heads, compared with the GPU's out [L][B][Hq][d] (numpy).  new_kv(l,
    b, h) -> (k, v) of the step's appended token, or None.  Returns (oracle
    seconds, KV bytes the units cover, worst max-abs, worst rel-L2)."""
    import numpy as np
    import torch
    import workloads as W
    from oracle import attention as OA, pool as OP
    G = w.Hq // w.Hkv
    import mixed_format_paged_amd as M
    layout = (w.Hq, w.Hkv, w.d)
    tb = M.mkv_tq3_page_bytes(layout) // w.Hkv
    fb = M.mkv_fp8_page_bytes(layout) // w.Hkv
    by_layer = {}
    for l, b, h in picks:
        by_layer.setdefault(l, []).append((b, h))
    t_oracle, bytes_done, worst, worst_rel = 0.0, 0, 0.0, 0.0
    for l, items in by_layer.items():
        vals = W.layer_values(w, st, l, device="cuda", requests={b for b, _ in items})
        for b, h in items:
            T = int(st.seq_lens[b])
            k = vals["k"][b][:, h].clone()
            v = vals["v"][b][:, h].clone()
            if new_kv is not None and T > 0:
                k[T - 1], v[T - 1] = new_kv(l, b, h)
            k, v = k.cpu().numpy(), v.cpu().numpy()
            q = vals["q"][b, h * G:(h + 1) * G].cpu().numpy()
            tiers = st.tiers[st.bt_offsets[b]:st.bt_offsets[b + 1]]
            is_tq3 = tiers == W.TIER_S
            t0 = time.perf_counter()
            K = OP.quantized_values(k, is_tq3, 1.0)
            V = OP.quantized_values(v, is_tq3, 1.0)
            o, _ = OA.decode_attention(q, K[:, None, :], V[:, None, :])
            t_oracle += time.perf_counter() - t0
            bytes_done += int(is_tq3.sum()) * tb + int((~is_tq3).sum()) * fb
            got = out[l, b, h * G:(h + 1) * G].astype(np.float64)
            worst = max(worst, float(np.abs(got - o).max()))
            worst_rel = max(worst_rel, float(np.linalg.norm(got - o) / max(np.linalg.norm(o), 1e-30)))
        del vals
        torch.cuda.empty_cache()
    return t_oracle, bytes_done, worst, worst_rel


def time_config(name, copies=1, passes=8, units=2):
    """One of the other workloads, single layer: the whole decode of one layer
    per pass (mkv_decode_attn: plan, partials, merge; for the demotion
    workload mkv_demote_pages of its aging pages first), captured in a HIP
    graph of `copies` passes, one per cache copy (a layer small enough for the
    last-level cache is held `copies` times over and the passes rotate through
    the copies, so no pass finds its pages cached), replayed `passes` times.
    Sampled outputs of copy 0 are checked against the oracle; for the
    demotion workload a sample of the demoted pages is compared byte for byte
    with the oracle's pack."""
    import numpy as np
    import torch
    import mixed_format_paged_amd as M
    import workloads as W
    from workloads.device_cache import DeviceWorkload
    from oracle import pool as OP
    w0 = W.WORKLOADS[name]
    w = W.scaled(w0, name=f"{name}-{copies}copies", L=copies) if copies > 1 else w0
    st = W.make_structure(w)
    t0 = time.time()
    dw = DeviceWorkload(w, st, "cuda")
    dw.step_demote()                     # the aging pages of the demotion workload (none elsewhere)
    torch.cuda.synchronize()
    build_s = time.time() - t0
    lay = (w.Hq, w.Hkv, w.d)
    bat = dw.batch()
    sm = 1.0 / math.sqrt(w.d)
    ws = torch.empty(M.mkv_decode_workspace_bytes(lay, w.B, dw.bt.numel(), 1), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.L, w.B, w.Hq, w.d), device="cuda")
    lse = torch.empty((w.L, w.B, w.Hq), device="cuda")
    q = [dw.q[l].contiguous() for l in range(w.L)]
    demote = dw.d_idx.numel() > 0

    def one(l):
        if demote:                        # rewrites the same TQ3 bytes every pass
            dw.cache.demote(l, dw.d_src, dw.d_dst)
        M.mkv_decode_attn(lay, dw.cache.pools[l], bat, q[l], sm, out[l], lse[l], ws)

    def replay_all():
        for l in range(w.L):
            one(l)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        replay_all()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        replay_all()
    graph.replay()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(passes + 1)]
    evs[0].record()
    for i in range(passes):
        graph.replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(evs[i].elapsed_time(evs[i + 1]) / w.L for i in range(passes))
    ms = evs[0].elapsed_time(evs[-1]) / passes / w.L
    status = M.mkv_workspace_status(ws)
    # the same passes with one plan for all copies (they share the tables), as
    # a model with several layers runs them: plan once, then partials + merge
    # per copy; per-layer time = pass time / copies
    ms_shared = None
    if w.L > 1:
        def shared_pass():
            M.mkv_decode_plan(lay, dw.cache.pools[0], bat, 1, ws)
            for l in range(w.L):
                if demote:
                    dw.cache.demote(l, dw.d_src, dw.d_dst)
                M.mkv_attend_partials(lay, [dw.cache.pools[l]], bat, q[l], sm, ws)
                M.mkv_merge(lay, 1, bat, out[l], lse[l], ws)
        with torch.cuda.stream(s):
            shared_pass()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph2 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph2):
            shared_pass()
        graph2.replay()
        torch.cuda.synchronize()
        a2, b2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a2.record()
        for _ in range(passes):
            graph2.replay()
        b2.record()
        torch.cuda.synchronize()
        ms_shared = a2.elapsed_time(b2) / passes / w.L
        status |= M.mkv_workspace_status(ws)
        del graph2
    # the demotion alone, same launch sizes
    dem = None
    if demote:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(5):
            dw.cache.demote(0, dw.d_src, dw.d_dst)
        b.record()
        torch.cuda.synchronize()
        dem_ms = a.elapsed_time(b) / 5
        n_dem = dw.d_src.numel()
        fb, tb = M.mkv_fp8_page_bytes(lay), M.mkv_tq3_page_bytes(lay)
        # a sample of the demoted pages against the oracle's pack, byte for byte
        pick = np.random.default_rng(9).choice(n_dem, 16, replace=False)
        src = dw.d_src[torch.as_tensor(pick, device="cuda")].cpu().numpy()
        dst = dw.d_dst[torch.as_tensor(pick, device="cuda")].cpu().numpy() - st.n_fp8
        pool = OP.Pool(w.Hkv, w.d, 16, 16, 1.0, 1.0)
        pool.fp8[:] = dw.cache.fp8[0][torch.as_tensor(src, dtype=torch.long, device="cuda")].cpu().numpy()
        OP.demote(pool, np.arange(16), 16 + np.arange(16))
        got = dw.cache.tq3[0][torch.as_tensor(dst, dtype=torch.long, device="cuda")].cpu().numpy()
        dem = {"pages": n_dem, "avg_ms": round(dem_ms, 5), "gbs": round(n_dem * (fb + tb) / (dem_ms * 1e-3) / 1e9, 2),
               "sample_bitexact_vs_oracle": bool(np.array_equal(got, pool.tq3))}
    n_t = int((st.tiers == W.TIER_S).sum())
    n_f = int(st.total_pages - n_t)
    layer_bytes = n_f * M.mkv_fp8_page_bytes(lay) + n_t * M.mkv_tq3_page_bytes(lay)
    picks = sorted({(0, int(b), int(h)) for b, h in zip(np.random.default_rng(21).integers(0, w.B, units),
                                                        np.random.default_rng(22).integers(0, w.Hkv, units))})
    _, _, worst, worst_rel = oracle_units(w, st, picks, out.cpu().numpy())
    res = {"workload": name, "batch": w0.B, "tokens": int(st.seq_lens.sum()), "layer_kv_bytes": layer_bytes,
           "cache_copies": w.L, "ms_per_layer": round(ms, 5), "p10_ms": round(per[int(0.1 * (passes - 1))], 5),
           "p90_ms": round(per[int(0.9 * (passes - 1))], 5),
           "kv_gbs": round(layer_bytes / (ms * 1e-3) / 1e9, 2),
           "pct_hbm_peak": round(100 * layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
           "tokens_per_s": round(w0.B / (ms * 1e-3), 2),
           "sampled_parity": {"units": len(picks), "max_abs": worst, "rel_l2": worst_rel,
                              "pass": bool(worst <= 2e-3 and worst_rel <= 1e-3)},
           "device_status": status, "build_s": round(build_s, 1)}
    if ms_shared is not None:
        res["plan_shared_by_copies"] = {"ms_per_layer": round(ms_shared, 5),
                                        "kv_gbs": round(layer_bytes / (ms_shared * 1e-3) / 1e9, 2),
                                        "note": "one plan per pass for all copies, as a model's layers share it"}
    if dem is not None:
        res["demote_then_decode"] = dict(dem, note="each pass demotes the aging pages, then decodes the layer")
    del dw, ws, out, lse, q, graph
    torch.cuda.empty_cache()
    return res


def stream_ceiling(nbytes=2 << 30, reps=10):
    """Streaming HBM rates measured in the same run, each over nbytes: a device
    copy (bytes read + written), a sum over the buffer (bytes read), and the
    decode kernels' page-staging loads alone (bytes read; mkv_stream_read)."""
    import torch
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    x.sum()
    torch.cuda.synchronize()
    res = {}
    for name, fn, moved in (("copy", lambda: y.copy_(x), 2 * nbytes), ("sum", lambda: x.sum(), nbytes)):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        res[f"{name}_gbs"] = round(moved / (ms * 1e-3) / 1e9, 1)
    # the page-staging loads of the decode kernels alone (mkv_stream_read)
    import mixed_format_paged_amd as M
    sink = torch.zeros(12 * 1024, dtype=torch.int32, device="cuda")
    M.mkv_stream_read(x, sink)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        M.mkv_stream_read(x, sink)
    b.record()
    torch.cuda.synchronize()
    moved = nbytes // 3584 * 3584
    res["staging_loads_gbs"] = round(moved / (a.elapsed_time(b) / reps * 1e-3) / 1e9, 1)
    del x, y, sink
    torch.cuda.empty_cache()
    res["bytes"] = nbytes
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(runner, units):
    """Time the CPU oracle on a bounded sample of the same step, and check the
    GPU's outputs for the sampled (layer, request, KV head) units against it;
    then one unit again with the oracle's numeric libraries held to one thread,
    and the oracle's FP8 -> TQ3 pack on a sample of pages."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import pool as OP
    w, st = runner.w, runner.st
    rng = np.random.default_rng(7)
    picks = [(int(rng.integers(w.L)), int(rng.integers(w.B)), int(rng.integers(w.Hkv))) for _ in range(units)]
    G = w.Hq // w.Hkv
    out = runner.out.cpu().numpy()
    new_kv = lambda l, b, h: (runner.k_new[l, b, 0, h], runner.v_new[l, b, 0, h])   # the step's appended token
    t_oracle, bytes_done, worst, worst_rel = oracle_units(w, st, picks, out, new_kv)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    with threadpool_limits(limits=1):
        t1, bytes1, _, _ = oracle_units(w, st, picks[:1], out, new_kv)
    # the pack, on 64 pages of random E4M3 bytes (no NaN codes)
    lay = runner.layout
    n = 64
    pool = OP.Pool(w.Hkv, w.d, n, n, 1.0, 1.0)
    raw = np.random.default_rng(3).integers(0, 254, pool.fp8.shape).astype(np.uint8)
    raw += (raw >= 0x7F).astype(np.uint8)
    pool.fp8[:] = raw
    t0 = time.perf_counter()
    OP.demote(pool, np.arange(n), n + np.arange(n))
    t_pack = time.perf_counter() - t0
    fb, tb = runner.M.mkv_fp8_page_bytes(lay), runner.M.mkv_tq3_page_bytes(lay)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {
        "value": round(bytes_done / t_oracle / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "cpu_model": cpu_model(), "cores_available": cores,
        "sample": (f"{units} (layer, request, KV head) units of the same step, each the oracle's "
                   f"quantise -> dequantise value path and fp64 attention for its {G} query heads over "
                   f"all {int(st.seq_lens[0])} tokens; {t_oracle:.1f} s of CPU time"),
        "tokens_per_s": round(w.B / (t_oracle / units * w.L * w.B * w.Hkv), 6),
        "kv_token_layers_per_s": round(units * int(st.seq_lens[0]) / t_oracle, 1),
        "one_thread": {"value": round(bytes1 / t1 / 1e9, 4), "unit": "GB/s", "sample": "the first unit above", "s": round(t1, 2)},
        "pack_fp8_to_tq3": {"pages": n, "s": round(t_pack, 3), "pages_per_s": round(n / t_pack, 1),
                            "gbs": round(n * (fb + tb) / t_pack / 1e9, 5),
                            "sample": "the oracle's pack of 64 pages of random E4M3 bytes (one layer)"},
        "parity_max_abs": worst, "parity_rel_l2": worst_rel,
    }


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (the library has no multi-GPU path); got --gpus {a.gpus}",
              file=sys.stderr)
        sys.exit(2)
    if a.copy_calibration:
        copy_calibration(a.copy_calibration, 5)
        return
    if a.pack_only:
        import types
        import torch
        import workloads as W
        import mixed_format_paged_amd as M
        w = W.WORKLOADS[a.workload]
        r = types.SimpleNamespace(torch=torch, M=M, layout=(w.Hq, w.Hkv, w.d))
        time_demote_pack(r, reps=1)
        ms, nbytes = time_demote_pack(r, reps=a.pack_only)
        print(json.dumps({"demote_pack_8192_pages": {"avg_us": round(ms * 1e3, 2), "bytes": nbytes,
                                                      "gbs": round(nbytes / ms / 1e6, 1),
                                                      "frac_of_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)},
                          "workload": w.name}), flush=True)
        return
    if a.item_trace:
        trace_lib = os.path.join(ROOT, "mixed_format_paged_amd", "libmkv_trace.so")
        if not os.path.exists(trace_lib):
            print("bench.py --item-trace needs the trace build: python -m mixed_format_paged_amd.build --item-trace",
                  file=sys.stderr)
            sys.exit(2)
        os.environ["MKV_LIB_PATH"] = trace_lib           # read when the package is first imported
    import torch
    import workloads as W
    w = W.WORKLOADS[a.workload]
    st = W.make_structure(w)
    print(f"[bench] building {w.name} cache on the GPU ...", file=sys.stderr, flush=True)
    r = Runner(w, st, kernel=a.kernel, fused_append=not a.separate_append)
    print(f"[bench] built in {r.build_s:.1f} s", file=sys.stderr, flush=True)
    if a.item_trace:
        for _ in range(3):
            r.step()
        torch.cuda.synchronize()
        rep_ = item_trace(r, a.item_trace)
        print("[bench] item trace of the partial-attention launch (us; p10, p50, p90, max over workgroups "
              "or waves; entry, stored: from the launch's first entry; the others per workgroup or wave)",
              file=sys.stderr, flush=True)
        for k, v in rep_.items():
            print(f"  {k:<26} {v}", flush=True)
        print(json.dumps({"item_trace": rep_, "workload": w.name}), flush=True)
        return
    if a.profile_steps:
        for _ in range(a.profile_steps):
            r.step()
        torch.cuda.synchronize()
        r.time_kernels(reps=5)
        time_materialize(r, reps=2)
        time_demote_pack(r, reps=2)
        time_lifecycle(r, reps=3)
        if a.kernel == "mfma":
            time_multi_query(r, reps=2)
        print(f"[bench] profile run: {a.profile_steps} eager steps done", file=sys.stderr, flush=True)
        return
    ms = r.time_steps(a.steps, a.warmup, graph=not a.no_graph)
    print(f"[bench] timed {a.steps} steps: {ms:.4f} ms/step", file=sys.stderr, flush=True)
    kv_bytes, tq3_bytes, tq3_bytes_layer = r.kv_bytes()
    layer_bytes = kv_bytes // w.L
    kt = r.time_kernels()
    k_avg, k_med = kt["partials"]
    mat_ms, mat_read, mat_written = time_materialize(r)
    dem_ms, dem_bytes = time_demote_pack(r)
    dem_s_ms, _ = time_demote_pack(r, scales=(0.37, 2.5))
    lc_ms, lc_demoted = time_lifecycle(r)
    # multi-query decode and rotated TQ3 run on the matrix-core kernels only
    mq_ms = time_multi_query(r, T=4) if a.kernel == "mfma" else None
    rot = time_rotated(r) if a.kernel == "mfma" else None
    traffic = recorded_traffic(w.name)
    status = r.M.mkv_workspace_status(r.ws)
    value = kv_bytes / (ms * 1e-3) / 1e9
    result = {
        "metric": "decode-attn KV GB/s + tokens/s at 2x59,008 ctx, 16 layers; % MI355X HBM peak",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16 mfma operands, f32 accumulate", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "seq_len": int(st.seq_lens[0]), "layers": w.L,
                   "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d, "page": 16,
                   "fp8_pages_per_request": int(st.n_pages[0] - (st.tiers[:st.n_pages[0]] == 2).sum()),
                   "tq3_pages_per_request": int((st.tiers[:st.n_pages[0]] == 2).sum()),
                   "kernel": a.kernel, "graph": not a.no_graph,
                   "append": "separate launch" if a.separate_append else "inside the attend launch"},
        "tokens_per_s": round(w.B / (ms * 1e-3), 2),
        "kv_token_layers_per_s": round(int(st.seq_lens.sum()) * w.L / (ms * 1e-3), 1),
        "ms_per_step_p10": round(r.step_p10, 5), "ms_per_step_median": round(r.step_median, 5),
        "ms_per_step_p90": round(r.step_p90, 5),
        "kv_bytes_per_step": kv_bytes,
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        # the same with the attention launches' measured HBM bytes (FETCH_SIZE + WRITE_SIZE per launch from
        # the committed counter summary, times the layers) in place of the algorithmic KV bytes
        "pct_hbm_peak_measured_bytes": (round(100 * traffic * w.L / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)
                                        if traffic else None),
        "device_status": status,
        "roofline": {"bound": "hbm", "kernel": "attend_kernel: FP8 + TQ3 partial attention, one layer",
                     "achieved": round(layer_bytes / (k_avg * 1e-3) / 1e9, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(layer_bytes / (k_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "avg_launch_ms": round(k_avg, 5), "median_launch_ms": round(k_med, 5),
                     "bytes_per_launch": layer_bytes},
        "merge_kernel": {"avg_launch_ms": round(kt["merge"][0], 5), "median_launch_ms": round(kt["merge"][1], 5)},
        # the dense BF16 shadow the decode path avoids, for one layer (all pages of every request)
        "materialize_dense_bf16": {"avg_ms_per_layer": round(mat_ms, 5), "bytes_read": mat_read,
                                   "bytes_written": mat_written,
                                   "gbs": round((mat_read + mat_written) / (mat_ms * 1e-3) / 1e9, 2),
                                   "frac_of_peak": round((mat_read + mat_written) / (mat_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                   "vs_decode_launch": round(mat_ms / k_avg, 3)},
        # the pack kernel alone at the 64 x 128 aging-page scale (random E4M3 pages, one layer)
        "demote_pack_8192_pages": {"avg_ms": round(dem_ms, 5), "bytes": dem_bytes,
                                   "gbs": round(dem_bytes / (dem_ms * 1e-3) / 1e9, 2),
                                   "frac_of_peak": round(dem_bytes / (dem_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        # the same pack with layer scales other than 1 (k_scale 0.37, v_scale 2.5)
        "demote_pack_8192_pages_scaled": {"avg_ms": round(dem_s_ms, 5), "scales": [0.37, 2.5],
                                          "frac_of_peak": round(dem_bytes / (dem_s_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        # mkv_lifecycle_step at a page boundary: FP8 pops, aging into TQ3 in all layers, table updates
        "lifecycle_step_page_boundary": {"avg_ms": round(lc_ms, 5), "layers": w.L,
                                         "pages_demoted_per_layer": lc_demoted},
        # each request's last 4 tokens as causal queries, one layer per call (plan + partials + merge)
        "multi_query_4_tokens": None if mq_ms is None else {
            "avg_ms_per_layer": round(mq_ms, 5), "query_tokens_per_s": round(w.B * 4 / (mq_ms * 1e-3), 1),
            "kv_gbs_per_query_token": round(4 * layer_bytes / (mq_ms * 1e-3) / 1e9, 2),
            "vs_single_query_launch": round(mq_ms / k_avg, 3)},
        "rotated_tq3_one_layer": rot,
        "stream_ceiling": stream_ceiling(),
    }
    result["roofline"]["frac_of_staging_load_ceiling"] = round(
        result["roofline"]["achieved"] / result["stream_ceiling"]["staging_loads_gbs"], 4)
    if not a.no_configs:
        # the other workloads of the benchmark set, one layer each: 8 requests
        # x 16,384 and one request of 131,072 tokens fit the last-level cache,
        # so they rotate through 8 cache copies
        others = []
        for name, copies in (("batch-8x16384", 8), ("ragged-32x4096-65536", 1), ("demote-64x32768", 1),
                             ("long-1x131072", 8)):
            print(f"[bench] {name} ...", file=sys.stderr, flush=True)
            others.append(time_config(name, copies))
        result["other_workloads"] = others
    if not a.no_control:
        del r
        torch.cuda.empty_cache()
        print("[bench] building the all-FP8 control ...", file=sys.stderr, flush=True)
        c = Runner(w, st, all_fp8=True, kernel=a.kernel, fused_append=not a.separate_append)
        c_ms = c.time_steps(a.steps, a.warmup, graph=not a.no_graph)
        c_bytes = c.kv_bytes()[0]
        result["control_all_fp8"] = {"ms_per_step": round(c_ms, 5), "kv_bytes_per_step": c_bytes,
                                     "kv_gbs": round(c_bytes / (c_ms * 1e-3) / 1e9, 2),
                                     "compression_vs_fp8": round(c_bytes / kv_bytes, 4),
                                     "compression_vs_bf16": round(2 * c_bytes / kv_bytes, 4),
                                     "throughput_vs_control": round(c_ms / ms, 4)}
        del c
        torch.cuda.empty_cache()
        r = None
    if not a.no_cpu_baseline:
        if r is None:
            r = Runner(w, st, kernel=a.kernel, fused_append=not a.separate_append)
            r.time_steps(1, 1, graph=not a.no_graph)
        print("[bench] timing the CPU oracle on a sample ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(r, a.cpu_units)
    print(json.dumps(result))


if __name__ == "__main__":
    main()

"""Page lifecycle of a decode step -- oracle side (test infrastructure only).

Minima-KV keeps Recent and protected Anchor pages in FP8, moves older
non-anchor pages to packed TQ3, and keeps every live-request page
addressable (arXiv 2608.23834, page 1, Abstract).  The pages give no
allocator.  Readings taken (the same ones include/mkv.h states):

* Free ids live in two stacks: fp8_free[0:tops[0]] holds free FP8 ids,
  tq3_free[0:tops[1]] free TQ3 ids (physical ids n_fp8 ...); a pop takes
  the entry just below the top.
* A decode step adds one token to every request.  A request whose seq_len is
  a multiple of 16 starts logical page n = seq_len / 16: it pops an FP8 id,
  whose tier becomes Recent.  Its page count is then n + 1; with a Recent
  window of R pages, logical page n - R leaves the window, and if its tier is
  Recent it pops a TQ3 id and is demoted in every layer (Anchor pages stay
  FP8; other tiers are left alone).
* Requests pop in request order; then each demoted page, in request order,
  gets its block-table entry switched to the TQ3 id (tier Stale), and its FP8
  id (tier free) is pushed onto the FP8 stack.
* All or nothing: a full block-table row, an id outside the pool, a tier that
  contradicts an id, too few free ids, or stack tops outside their arrays
  leave everything unchanged and return status bits.

Release: every live page of the listed requests (in list order, then
logical order) is pushed onto its format's stack, its tier becomes free, and
the request's seq_len becomes 0.
"""
import numpy as np

from .layout import PAGE
from .pool import demote, TIER_R, TIER_S, TIER_FREE

BAD_PAGE_ID, BAD_TIER, BAD_SEQ_LEN, NO_FREE_PAGE = 1, 2, 4, 8


class Tables:
    """Mutable per-step state shared by all layers."""

    def __init__(self, bt_offsets, bt_pages, seq_lens, tier, fp8_free, tq3_free, tops):
        self.bt_offsets = np.asarray(bt_offsets, dtype=np.int64)
        self.bt_pages = np.asarray(bt_pages, dtype=np.int64).copy()
        self.seq_lens = np.asarray(seq_lens, dtype=np.int64).copy()
        self.tier = tier                                  # the pools' shared tier array
        self.fp8_free = np.asarray(fp8_free, dtype=np.int64).copy()
        self.tq3_free = np.asarray(tq3_free, dtype=np.int64).copy()
        self.tops = [int(tops[0]), int(tops[1])]


def step(pools, t, recent_pages):
    """One decode step's lifecycle on every layer's pool.  Returns status bits."""
    n_fp8, n_tq3 = pools[0].n_fp8, pools[0].n_tq3
    B = len(t.seq_lens)
    cap = len(t.bt_pages)
    top_f, top_t = t.tops
    err = 0
    plan = []                          # per request: (new_page, demote, aged index, aged id)
    for b in range(B):
        lo, hi, sl = int(t.bt_offsets[b]), int(t.bt_offsets[b + 1]), int(t.seq_lens[b])
        if sl < 0 or lo < 0 or hi < lo or hi > cap:
            err |= BAD_SEQ_LEN
            plan.append(None)
            continue
        n = -(-sl // PAGE)
        if n > hi - lo:
            err |= BAD_SEQ_LEN
            plan.append(None)
            continue
        if sl % PAGE != 0:
            plan.append((False, False, -1, -1))
            continue
        if n + 1 > hi - lo:
            err |= BAD_SEQ_LEN
            plan.append(None)
            continue
        aged = n - recent_pages
        if aged < 0:
            plan.append((True, False, -1, -1))
            continue
        aid = int(t.bt_pages[lo + aged])
        if not 0 <= aid < n_fp8 + n_tq3:
            err |= BAD_PAGE_ID
            plan.append(None)
            continue
        dem = int(t.tier[aid]) == TIER_R
        if dem and aid >= n_fp8:
            err |= BAD_TIER
            plan.append(None)
            continue
        plan.append((True, dem, aged, aid))
    stacks_ok = 0 <= top_f <= n_fp8 and 0 <= top_t <= n_tq3
    # the ids the pops would take, in request order
    pops_f, pops_t = [], []
    for p in plan:
        if p is None:
            continue
        if p[0]:
            k = len(pops_f)
            if stacks_ok and k < top_f:
                pid = int(t.fp8_free[top_f - 1 - k])
                if not 0 <= pid < n_fp8:
                    err |= BAD_PAGE_ID
                elif int(t.tier[pid]) != TIER_FREE:
                    err |= BAD_TIER
            pops_f.append(k)
        if p[1]:
            k = len(pops_t)
            if stacks_ok and k < top_t:
                pid = int(t.tq3_free[top_t - 1 - k])
                if not n_fp8 <= pid < n_fp8 + n_tq3:
                    err |= BAD_PAGE_ID
                elif int(t.tier[pid]) != TIER_FREE:
                    err |= BAD_TIER
            pops_t.append(k)
    nf, nt = len(pops_f), len(pops_t)
    if not stacks_ok or nf > top_f or nt > top_t or top_f - nf + nt > n_fp8:
        err |= NO_FREE_PAGE
    if err:
        return err
    # apply: pops in request order
    kf = kt = 0
    demotions = []                     # (src FP8 id, dst TQ3 id, block-table entry)
    for b in range(B):
        new_page, dem, aged, aid = plan[b]
        lo, sl = int(t.bt_offsets[b]), int(t.seq_lens[b])
        if new_page:
            pid = int(t.fp8_free[top_f - 1 - kf])
            kf += 1
            t.bt_pages[lo + sl // PAGE] = pid
            t.tier[pid] = TIER_R
        if dem:
            dst = int(t.tq3_free[top_t - 1 - kt])
            kt += 1
            demotions.append((aid, dst, lo + aged))
        t.seq_lens[b] = sl + 1
    top_f -= kf
    top_t -= kt
    # demote in every layer, switch the entries, free the FP8 ids
    for i, (src, dst, entry) in enumerate(demotions):
        for pool in pools:
            demote(pool, [src], [dst])
        t.bt_pages[entry] = dst
        t.tier[dst] = TIER_S
        t.tier[src] = TIER_FREE
        t.fp8_free[top_f + i] = src
    t.tops = [top_f + len(demotions), top_t]
    return 0


def release(pool, t, requests):
    """Return every live page of the listed requests to the free stacks."""
    n_fp8, n_tq3 = pool.n_fp8, pool.n_tq3
    B = len(t.seq_lens)
    cap = len(t.bt_pages)
    err = 0
    need_f = need_t = 0
    for b in requests:
        b = int(b)
        if not 0 <= b < B:
            err |= BAD_SEQ_LEN
            continue
        lo, hi, sl = int(t.bt_offsets[b]), int(t.bt_offsets[b + 1]), int(t.seq_lens[b])
        n = -(-sl // PAGE)
        if sl < 0 or lo < 0 or hi < lo or hi > cap or n > hi - lo:
            err |= BAD_SEQ_LEN
            continue
        for lp in range(n):
            pid = int(t.bt_pages[lo + lp])
            if not 0 <= pid < n_fp8 + n_tq3:
                err |= BAD_PAGE_ID
            elif int(t.tier[pid]) == TIER_FREE:
                err |= BAD_TIER
            elif pid < n_fp8:
                need_f += 1
            else:
                need_t += 1
    top_f, top_t = t.tops
    if top_f < 0 or top_t < 0 or top_f + need_f > n_fp8 or top_t + need_t > n_tq3:
        err |= NO_FREE_PAGE
    if err:
        return err
    for b in requests:
        b = int(b)
        lo = int(t.bt_offsets[b])
        for lp in range(-(-int(t.seq_lens[b]) // PAGE)):
            pid = int(t.bt_pages[lo + lp])
            if pid < n_fp8:
                t.fp8_free[top_f] = pid
                top_f += 1
            else:
                t.tq3_free[top_t] = pid
                top_t += 1
            t.tier[pid] = TIER_FREE
        t.seq_lens[b] = 0
    t.tops = [top_f, top_t]
    return 0

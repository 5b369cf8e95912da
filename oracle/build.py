"""Build a layer's cache the way the method's lifecycle does -- oracle side.

Test infrastructure only.  Every token is first written to an FP8 page
(Recent); pages that are stale are then demoted to TQ3 and their FP8 slot is
freed, which is the "older non-anchor pages move to packed TQ3" step of the
pages (arXiv 2608.23834, page 1, Abstract).  A workload's aging pages (if
any) stay FP8 here and are demoted by `step_demote` during the timed step.
"""
import numpy as np

from .pool import Pool, append, demote, TIER_R, TIER_S, TIER_FREE


def build_layer(w, st, k_list, v_list, k_scale=1.0, v_scale=1.0, signs=None):
    """Returns (pool, bt_pages) for the state before the step's own demotion.
    signs: rotated TQ3 pages (oracle/rotation.py) with this sign vector."""
    pool = Pool(w.Hkv, w.d, st.n_fp8, st.n_tq3, k_scale, v_scale, signs=signs)
    bt = st.staging_ids.astype(np.int64).copy()
    pool.tier[bt] = TIER_R
    for b in range(w.B):
        off = np.array([0, st.n_pages[b]])
        pages = bt[st.bt_offsets[b]:st.bt_offsets[b + 1]]
        append(pool, np.asarray(k_list[b])[None], np.asarray(v_list[b])[None], off, pages, [0])
    _demote_entries(pool, st, bt, st.build_entries)
    fp8_entries = np.nonzero(st.tiers != TIER_S)[0]
    pool.tier[bt[fp8_entries]] = st.tiers[fp8_entries]          # R or A
    return pool, bt


def step_demote(pool, st, bt):
    """The step's demotion of aging pages (FP8 -> TQ3); updates bt and tiers in place."""
    _demote_entries(pool, st, bt, st.demote_entries)


def _demote_entries(pool, st, bt, entries):
    if len(entries) == 0:
        return
    src = bt[entries].copy()
    dst = st.final_ids[entries].astype(np.int64)
    demote(pool, src, dst)
    bt[entries] = dst
    pool.tier[dst] = TIER_S
    pool.tier[src] = TIER_FREE

"""Seeded synthetic inputs for mixed FP8 / TQ3 paged decode attention.

Shared by the oracle side (tests) and the HIP side (tests, bench).  This
module holds NO arithmetic of the method: it only draws lengths, tier
assignments, physical page placement and fp32 source values.  Quantisation,
packing and attention happen on each side separately.

Shapes follow the pages' direct-decode canary (two requests of 59,008
tokens, 16 full-attention layers: arXiv 2608.23834, page 1, Abstract) and a
family of synthetic decode batches around it.  No public dataset is used:
every value is drawn from the seeded generators below.

Draw order per workload: lengths, anchors, pool permutation (numpy
default_rng(seed)), then per layer the outlier channels / per-channel
log-normal scales (numpy) and the bulk N(0, 1) tensors (torch generator on
the requested device, seeded from (seed, layer)).  The bulk tensors differ
between devices; both sides always consume the same tensor (copied where
needed), never two independent draws.
"""
from dataclasses import dataclass, field
import numpy as np

PAGE = 16
TIER_R, TIER_A, TIER_S, TIER_FREE = 0, 1, 2, 0xFF


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    L: int
    Hq: int
    Hkv: int
    d: int
    lengths: tuple            # ("fixed", n), ("uniform", lo, hi) or ("list", (n_0, ..., n_B-1))
    recent_tokens: int
    fixed_anchor_pages: int
    random_anchor_frac: float
    values: str               # "outlier" or "lognormal"
    seed: int
    aging_pages: int = 0      # pages demoted FP8 -> TQ3 during the step


WORKLOADS = {
    w.name: w for w in [
        # 1 request x 1,024 tokens, d = 128: pages 0-1 anchor, last 4 recent, 58 TQ3.
        Workload("tiny-1x1024-d128", 1, 1, 24, 4, 128, ("fixed", 1024), 64, 2, 0.0, "outlier", 0),
        # 8 requests x 16,384 tokens, one layer: recent 512 tokens, anchors first 4 + 2 %.
        Workload("batch-8x16384", 8, 1, 24, 4, 256, ("fixed", 16384), 512, 4, 0.02, "lognormal", 1),
        # the canary shape: 2 x 59,008 tokens, 16 layers, recent 1,024 tokens + 8 anchor pages.
        Workload("canary-2x59008-16L", 2, 16, 24, 4, 256, ("fixed", 59008), 1024, 8, 0.0, "outlier", 2),
        # 32 ragged requests, lengths uniform in [4,096, 65,536], 3 % random anchors.
        Workload("ragged-32x4096-65536", 32, 1, 24, 4, 256, ("uniform", 4096, 65536), 512, 0, 0.03, "lognormal", 3),
        # 64 x 32,768 tokens; 128 pages per request age FP8 -> TQ3 in the step, then decode.
        Workload("demote-64x32768", 64, 1, 24, 4, 256, ("fixed", 32768), 512, 4, 0.0, "lognormal", 4, aging_pages=128),
        # one 131,072-token request split over the whole GPU (multi-level merge).
        Workload("long-1x131072", 1, 1, 24, 4, 256, ("fixed", 131072), 512, 4, 0.02, "lognormal", 4),
    ]
}


def scaled(w, name=None, **kw):
    """A smaller variant of a workload (same structure rules) for fast tests."""
    from dataclasses import replace
    return replace(w, name=name or (w.name + "-small"), **kw)


@dataclass
class Structure:
    seq_lens: np.ndarray        # int32 [B]
    n_pages: np.ndarray         # int32 [B]
    bt_offsets: np.ndarray      # int32 [B + 1]
    tiers: np.ndarray           # uint8 [total] logical tier per block-table entry (after the step's demotion)
    staging_ids: np.ndarray     # int32 [total] FP8 slot each logical page is first written to
    final_ids: np.ndarray       # int32 [total] physical id in the decoded cache
    n_fp8: int
    n_tq3: int
    demote_entries: np.ndarray  # int64 [n] block-table entries demoted during the step
    build_entries: np.ndarray   # int64 [m] entries demoted while building the cache (before the step)

    @property
    def total_pages(self):
        return int(self.bt_offsets[-1])


def make_structure(w):
    rng = np.random.default_rng(w.seed)
    # 1. lengths
    if w.lengths[0] == "fixed":
        lens = np.full(w.B, w.lengths[1], dtype=np.int64)
    elif w.lengths[0] == "list":
        lens = np.array(w.lengths[1], dtype=np.int64)
        assert len(lens) == w.B
    else:
        lens = rng.integers(w.lengths[1], w.lengths[2] + 1, size=w.B)
    n_pages = -(-lens // PAGE)
    offsets = np.zeros(w.B + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(n_pages)
    total = int(offsets[-1])
    # 2. tiers: recent window, fixed anchors, random anchors, aging pages
    tiers = np.full(total, TIER_S, dtype=np.uint8)
    aging = np.zeros(total, dtype=bool)
    recent_pages = w.recent_tokens // PAGE
    for b in range(w.B):
        n = int(n_pages[b])
        t = tiers[offsets[b]:offsets[b + 1]]
        ag = aging[offsets[b]:offsets[b + 1]]
        first_recent = max(0, n - recent_pages)
        fixed = list(range(min(w.fixed_anchor_pages, first_recent)))
        t[fixed] = TIER_A
        if w.random_anchor_frac > 0:
            k = int(round(w.random_anchor_frac * n))
            cand = np.setdiff1d(np.arange(first_recent), np.array(fixed, dtype=np.int64))
            k = min(k, len(cand))
            t[rng.choice(cand, size=k, replace=False)] = TIER_A
        if w.aging_pages:
            lo = max(0, first_recent - w.aging_pages)
            for lp in range(lo, first_recent):
                if t[lp] == TIER_S:
                    ag[lp] = True
        t[first_recent:] = TIER_R
    # 3. pool permutation: every page gets an FP8 staging slot; TQ3 pages a TQ3 slot.
    n_fp8 = total
    staging = rng.permutation(total).astype(np.int64)
    is_tq3 = tiers == TIER_S
    n_tq3 = int(is_tq3.sum())
    tq3_slot = np.full(total, -1, dtype=np.int64)
    tq3_slot[is_tq3] = n_fp8 + rng.permutation(n_tq3)
    final = np.where(is_tq3, tq3_slot, staging)
    demote_entries = np.nonzero(aging)[0]
    build_entries = np.nonzero(is_tq3 & ~aging)[0]
    return Structure(lens.astype(np.int32), n_pages.astype(np.int32), offsets.astype(np.int32),
                     tiers, staging.astype(np.int32), final.astype(np.int32), n_fp8, n_tq3,
                     demote_entries, build_entries)


def _layer_seed(w, layer):
    return int(w.seed) * 1_000_003 + int(layer) * 7919 + 17


def layer_values(w, st, layer, device="cpu", requests=None):
    """fp32 source values for one layer.

    Returns dict(k=[T_b][Hkv][d] per request, v=..., q=[B][Hq][d]) as torch
    tensors on `device`.  Value recipes:
      "outlier":   q, K, V ~ N(0, 1); for each KV head 4 distinct channels are
                   multiplied by 8 in K, V and in q of the heads of that group.
      "lognormal": K, V = z * exp(0.5 * xi[h, c]), z ~ N(0, 1), xi ~ N(0, 1)
                   per (head, channel), separately for K and V; q ~ N(0, 1).
    `requests` restricts generation to a subset (values of the others are
    still drawn in the same order, so a subset equals the full draw).
    """
    import torch
    rng = np.random.default_rng(_layer_seed(w, layer))
    G = w.Hq // w.Hkv
    kmul = np.ones((w.Hkv, w.d), dtype=np.float32)
    vmul = np.ones((w.Hkv, w.d), dtype=np.float32)
    qmul = np.ones((w.Hq, w.d), dtype=np.float32)
    if w.values == "outlier":
        for h in range(w.Hkv):
            ch = rng.choice(w.d, size=4, replace=False)
            kmul[h, ch] = 8.0
            vmul[h, ch] = 8.0
            qmul[h * G:(h + 1) * G, ch[None, :]] = 8.0
    elif w.values == "lognormal":
        kmul = np.exp(0.5 * rng.standard_normal((w.Hkv, w.d))).astype(np.float32)
        vmul = np.exp(0.5 * rng.standard_normal((w.Hkv, w.d))).astype(np.float32)
    else:
        raise ValueError(w.values)
    g = torch.Generator(device=device)
    g.manual_seed(_layer_seed(w, layer))
    q = torch.randn((w.B, w.Hq, w.d), generator=g, device=device, dtype=torch.float32)
    q = q * torch.as_tensor(qmul, device=device)
    km = torch.as_tensor(kmul, device=device)
    vm = torch.as_tensor(vmul, device=device)
    ks, vs = [], []
    for b in range(w.B):
        T = int(st.seq_lens[b])
        kb = torch.randn((T, w.Hkv, w.d), generator=g, device=device, dtype=torch.float32)
        vb = torch.randn((T, w.Hkv, w.d), generator=g, device=device, dtype=torch.float32)
        if requests is None or b in requests:
            ks.append(kb * km)
            vs.append(vb * vm)
        else:
            ks.append(None)
            vs.append(None)
        del kb, vb
    return dict(k=ks, v=vs, q=q)

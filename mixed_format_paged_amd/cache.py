"""Device memory for a mixed FP8 / TQ3 paged cache (torch tensors as plumbing).

A PagedCache holds, per layer, one FP8 slab and one TQ3 slab, plus one tier
map shared by all layers; PoolDesc views of them are passed to libmkv.  Every
byte of page data is written by libmkv kernels (mkv_append, mkv_demote_pages);
this module only allocates memory and updates block-table entries and tier
bytes, which the caller owns (arXiv 2608.23834, page 1, Abstract: pages move
from FP8 to packed TQ3 while staying addressable).
"""
import torch

from . import (Layout, TIER_FREE, TIER_STALE, make_pool, mkv_append, mkv_demote_pages,
               mkv_fp8_page_bytes, mkv_tq3_page_bytes, _layout)

APPEND_MAX = 65520        # tokens per mkv_append call when filling a request (a whole number of pages)


class PagedCache:
    def __init__(self, layout, n_layers, n_fp8, n_tq3, device="cuda", k_scale=1.0, v_scale=1.0, tq3_signs=None):
        """tq3_signs: None, or one device int8 [head_dim] tensor per layer
        (rotated TQ3 pages in that layer; None entries: plain TQ3)."""
        self.layout = _layout(layout)
        self.n_layers, self.n_fp8, self.n_tq3 = int(n_layers), int(n_fp8), int(n_tq3)
        fb, tb = mkv_fp8_page_bytes(self.layout), mkv_tq3_page_bytes(self.layout)
        self.fp8 = [torch.zeros((max(1, n_fp8), fb), dtype=torch.uint8, device=device) for _ in range(n_layers)]
        self.tq3 = [torch.zeros((max(1, n_tq3), tb), dtype=torch.uint8, device=device) for _ in range(n_layers)]
        self.tier = torch.full((n_fp8 + n_tq3,), TIER_FREE, dtype=torch.uint8, device=device)
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)
        self.signs = list(tq3_signs) if tq3_signs is not None else [None] * n_layers
        self.pools = [make_pool(self.fp8[l], self.tq3[l], self.tier, n_fp8, n_tq3, k_scale, v_scale, self.signs[l])
                      for l in range(n_layers)]

    @property
    def kv_bytes_per_layer(self):
        return self.fp8[0].numel() + self.tq3[0].numel()

    def append(self, layer, k, v, bt_offsets, bt_pages, pos, counts=None, stream=None):
        mkv_append(self.layout, self.pools[layer], k, v, bt_offsets, bt_pages, pos, counts, stream)

    def demote(self, layer, src_fp8, dst_tq3, stream=None):
        mkv_demote_pages(self.layout, self.pools[layer], src_fp8, dst_tq3, stream)

    def fill_request(self, layer, k, v, fp8_pages):
        """Write one request's tokens k, v [T][Hkv][d] (fp32, device) from
        position 0 onward onto the FP8 pages `fp8_pages` (int32, device), in
        appends of at most APPEND_MAX tokens (mkv_append takes up to 65535)."""
        n_pages = fp8_pages.numel()
        dev = k.device
        offs = torch.tensor([0, n_pages], dtype=torch.int32, device=dev)
        pages = fp8_pages.contiguous()
        for t0 in range(0, k.shape[0], APPEND_MAX):
            t1 = min(k.shape[0], t0 + APPEND_MAX)
            pos = torch.tensor([t0], dtype=torch.int32, device=dev)
            self.append(layer, k[t0:t1].unsqueeze(0).contiguous(), v[t0:t1].unsqueeze(0).contiguous(), offs,
                        pages, pos)

    def retier_demoted(self, src_fp8, dst_tq3):
        """After demotion on every layer: dst pages become Stale, src slots free."""
        self.tier[dst_tq3.long()] = TIER_STALE
        self.tier[src_fp8.long()] = TIER_FREE

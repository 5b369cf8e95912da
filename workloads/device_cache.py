"""Build a workload's cache on the GPU through libmkv (no method arithmetic here).

Same lifecycle as the oracle's build: every token is appended to an FP8
staging page with mkv_append, stale pages are demoted with mkv_demote_pages,
then block-table entries and tier bytes are rewritten (caller-owned state).
Values come from workloads.layer_values on the device.
"""
import numpy as np
import torch

from . import layer_values, TIER_S
from mixed_format_paged_amd import make_batch
from mixed_format_paged_amd.cache import PagedCache


class DeviceWorkload:
    def __init__(self, w, st, device="cuda", layers=None, keep_values=False, gen_device=None, spare_tq3=0,
                 tq3_signs=None, k_scale=1.0, v_scale=1.0, value_fn=None):
        """gen_device: where the fp32 values are drawn (default: `device`); tests
        draw on the CPU so the oracle can consume the very same tensors.
        spare_tq3: extra TQ3 slots after the workload's own (ids n_fp8 + n_tq3 ...).
        tq3_signs: None, or per built layer an int8 [d] sign vector (numpy or
        None): that layer's TQ3 pages are rotated TQ3.
        k_scale, v_scale: the pools' FP8 scales (every layer).
        value_fn(vals, layer) -> vals: applied to each layer's drawn values
        before they are written (tests use it to put values in other units)."""
        self.w, self.st = w, st
        n_layers = w.L if layers is None else len(layers)
        self.layers = list(range(w.L)) if layers is None else list(layers)
        signs = None if tq3_signs is None else [
            None if s is None else torch.as_tensor(np.asarray(s, dtype=np.int8), device=device) for s in tq3_signs]
        self.cache = PagedCache((w.Hq, w.Hkv, w.d), n_layers, st.n_fp8, st.n_tq3 + spare_tq3, device,
                                k_scale=k_scale, v_scale=v_scale, tq3_signs=signs)
        dev = device
        self.bt = torch.as_tensor(st.staging_ids, dtype=torch.int32, device=dev).clone()
        self.bt_offsets = torch.as_tensor(st.bt_offsets, dtype=torch.int32, device=dev)
        self.seq_lens = torch.as_tensor(st.seq_lens, dtype=torch.int32, device=dev)
        self.cache.tier[self.bt.long()] = 0          # every staging page starts Recent
        self.q = torch.empty((n_layers, w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
        self.values = [] if keep_values else None
        b_src = torch.as_tensor(st.staging_ids[st.build_entries], dtype=torch.int32, device=dev)
        b_dst = torch.as_tensor(st.final_ids[st.build_entries], dtype=torch.int32, device=dev)
        for li, layer in enumerate(self.layers):
            vals = layer_values(w, st, layer, device=gen_device or dev)
            if value_fn is not None:
                vals = value_fn(vals, layer)
            self.q[li] = vals["q"].to(dev)
            for b in range(w.B):
                pages = self.bt[int(st.bt_offsets[b]):int(st.bt_offsets[b + 1])]
                if int(st.seq_lens[b]) > 0:
                    self.cache.fill_request(li, vals["k"][b].to(dev), vals["v"][b].to(dev), pages)
            if len(st.build_entries):
                self.cache.demote(li, b_src, b_dst)
            if keep_values:
                self.values.append(vals)
            else:
                del vals
        if len(st.build_entries):
            idx = torch.as_tensor(st.build_entries, dtype=torch.long, device=dev)
            self.bt[idx] = b_dst
            self.cache.retier_demoted(b_src, b_dst)
        fp8_entries = np.nonzero(st.tiers != TIER_S)[0]
        ent = torch.as_tensor(fp8_entries, dtype=torch.long, device=dev)
        self.cache.tier[self.bt[ent].long()] = torch.as_tensor(st.tiers[fp8_entries], device=dev)
        # the step's own demotion (aging pages), if any, is left to step_demote()
        self.d_src = torch.as_tensor(st.staging_ids[st.demote_entries], dtype=torch.int32, device=dev)
        self.d_dst = torch.as_tensor(st.final_ids[st.demote_entries], dtype=torch.int32, device=dev)
        self.d_idx = torch.as_tensor(st.demote_entries, dtype=torch.long, device=dev)

    def batch(self):
        return make_batch(self.bt_offsets, self.bt, self.seq_lens)

    def step_demote(self):
        """Demote the aging pages on every layer and retier them."""
        if self.d_idx.numel() == 0:
            return
        for li in range(len(self.layers)):
            self.cache.demote(li, self.d_src, self.d_dst)
        self.bt[self.d_idx] = self.d_dst
        self.cache.retier_demoted(self.d_src, self.d_dst)

"""Helpers shared by the GPU tests: build the same workload on both sides.

The oracle side builds its byte pool with oracle.build from CPU-drawn values;
the HIP side builds its cache with libmkv kernels from the very same values
(copied to the GPU).  Nothing on the oracle side comes from the HIP path.
"""
import math

import numpy as np
import torch

import workloads as W
from oracle import attention as OA, build as OB, pool as OP

ATOL = 2e-3          # max |o_gpu - o_ref|
RTOL_L2 = 1e-3       # ||o_gpu - o_ref|| / ||o_ref||
LSE_ATOL = 1e-3


def need_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def oracle_side(w, st, layer_vals, signs=None, k_scale=1.0, v_scale=1.0):
    """Oracle pools, block tables and decode outputs for every layer
    (signs: per layer None or the sign vector of rotated TQ3 pages;
    k_scale, v_scale: the pools' FP8 scales)."""
    res = []
    for li, vals in enumerate(layer_vals):
        k = [None if x is None else x.cpu().numpy() for x in vals["k"]]
        v = [None if x is None else x.cpu().numpy() for x in vals["v"]]
        pool, bt = OB.build_layer(w, st, k, v, k_scale, v_scale, signs=None if signs is None else signs[li])
        OB.step_demote(pool, st, bt)
        o, lse = OA.decode_batch(pool, vals["q"].cpu().numpy(), st.bt_offsets, bt, st.seq_lens)
        res.append((pool, bt, o, lse))
    return res


def compare(o_gpu, o_ref, lse_gpu=None, lse_ref=None, what=""):
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    err = np.abs(o_gpu - o_ref)
    max_abs = float(err.max()) if err.size else 0.0
    den = float(np.linalg.norm(o_ref))
    rel = float(np.linalg.norm(o_gpu - o_ref)) / den if den > 0 else float(np.linalg.norm(o_gpu))
    msg = f"{what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}"
    assert max_abs <= ATOL, msg
    assert rel <= RTOL_L2, msg
    if lse_gpu is not None:
        lg = np.asarray(lse_gpu, dtype=np.float64)
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isneginf(lg), np.isneginf(lse_ref)), what + ": -inf pattern of lse"
        if fin.any():
            le = float(np.abs(lg[fin] - lse_ref[fin]).max())
            assert le <= LSE_ATOL, f"{what}: lse err {le:.3e}"
    return max_abs, rel


def in_units(k_scale, v_scale, seed=0, sat_frac=0.003):
    """value_fn for DeviceWorkload: K in units of k_scale and V in units of
    v_scale (the values times the scale, so their FP8 codes are those of the
    unit-scale values), and a fraction sat_frac of the V entries set to
    +-440 v_scale, near the top of the FP8 range, so TQ3 V scales reach
    fp16(448 v_scale / 3).  q is divided by k_scale, so the scores keep the
    size they have at unit scale (scores of hundreds of nats would make the
    fp32 rounding of the scores alone move the outputs past the bar)."""
    import torch

    def fn(vals, layer):
        g = torch.Generator()
        g.manual_seed(seed * 1000 + layer)
        vs = []
        for x in vals["v"]:
            if x is None:
                vs.append(None)
                continue
            y = x * v_scale
            hit = torch.rand(y.shape, generator=g) < sat_frac
            sign = torch.where(torch.rand(y.shape, generator=g) < 0.5, -1.0, 1.0)
            vs.append(torch.where(hit.to(y.device), (sign * 440.0 * v_scale).to(y.device), y))
        ks = [None if x is None else x * k_scale for x in vals["k"]]
        return dict(k=ks, v=vs, q=vals["q"] / k_scale)
    return fn

"""Shared helpers of the GPU parity tests (imported by tests/test_gpu_*.py)."""
import os
import sys

import numpy as np
import pytest

import datagen as dg
import oracle as orc

# Tolerances on row_err (max over rows of ||y - ref||_inf / ||ref||_inf):
# 1e-5 for fp32 and 2e-2 for bf16 with fp32 accumulation
TOL = {"f32": 1e-5, "bf16": 2e-2}


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from token_moe_amd import tmx
    tmx.load_library()   # fails loudly if the HIP library is missing


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def to_dev(wl, a):
    from token_moe_amd import runner
    return runner.host_tensor(wl, a).cuda()


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def row_err(y, yref):
    """max over rows of ||y - yref||_inf / ||yref||_inf (rows = last axis)."""
    y = np.asarray(y, np.float64)
    yref = np.asarray(yref, np.float64)
    num = np.max(np.abs(y - yref), axis=-1)
    den = np.max(np.abs(yref), axis=-1)
    return float(np.max(num / den))


_CACHE = {}


def context(key, wl, B_max=None, banks=None):
    """(ctx, banks, weight source) for a workload, cached per key."""
    if key in _CACHE:
        return _CACHE[key]
    from token_moe_amd import runner
    if banks is None:
        banks = dg.weight_banks(wl)
    ctx = runner.make_context(wl, banks, B_max=B_max)
    out = (ctx, banks, dg.WeightSource(wl, banks))
    _CACHE[key] = out
    return out


def drop(key):
    v = _CACHE.pop(key, None)
    if v is not None:
        v[0].close()


def sample_rows(B, n, seed=0):
    """Fixed seeded subset of sample rows, always including the first and last."""
    rng = np.random.default_rng(1000 + seed)
    n = min(n, B)
    rows = set(rng.choice(B, size=n, replace=False).tolist())
    rows.update({0, B - 1})
    return np.array(sorted(rows))


def oracle_sublayer(wl, ws, layer, sub, x_rows, resid_rows=None, extra_rows=None):
    """Oracle of one sub-layer in block layout [n, T, D] (layer is 1-based)."""
    rho = wl.bf16_values
    mx = wl.dtype == "mxfp8"
    if sub == 0:
        Hm = orc.mix(x_rows, wl.H)
        return orc.revert(orc.sublayer_positions(Hm, Hm, wl, layer, 0, ws, None, rho, None, mx), wl.T)
    return orc.sublayer_positions(x_rows, resid_rows, wl, layer, 1, ws, extra_rows, rho, None, mx)

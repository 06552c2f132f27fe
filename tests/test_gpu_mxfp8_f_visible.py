"""MXFP8 parity with F visible, at the full workload shapes and launch
configurations (the MXFP8 counterpart of test_gpu_f_visible.py).

The workloads draw every down matrix at full scale (down_scale = 1), so the
FFN output F is as large as the residual and a wrong or missing F cannot
hide under it. Compared rows: one seeded row from every row tile of the
batch (second and later tiles of each persistent workgroup included; each
sample row holds all positions).

Bounds (see test_gpu_mxfp8.py): the kernels and the oracle take the same
quantisation decisions from fp32 values that differ in their last bits, so
an E4M3 code or a block exponent can flip, moving a value by at most half a
step of the coarser grid, 2^-4 of itself. Rows are held to 2^-4 and the
median row to 5e-3 (a layout or scale error moves every row). MoE
sub-layers are compared teacher-forced on the GPU's choice of experts, once
that choice is checked against the oracle's routing."""
import numpy as np
import pytest

import datagen as dg
from gpu_common import (check_routing, context, drop, oracle_sublayer, require_gpu, route_gpu, route_oracle,
                        say, stream, tile_rows, to_dev, to_np)

pytestmark = pytest.mark.gpu

TOL_F = 2.0 ** -4
TOL_F_MEDIAN = 5e-3


def visible(wid):
    wl = dg.WORKLOADS[wid]
    return wl.with_(name=wl.name + "_mx_fvis", dtype="mxfp8", down_scale=1.0)


def _ctx(wid):
    return context(f"mxfv{wid}", visible(wid))


def per_row(y, ref):
    """Row-normwise error over the elements the oracle evaluated (NaN marks
    positions left out; rows with none come back NaN)."""
    ok = ~np.isnan(ref)
    d = np.where(ok, np.abs(y - ref), -np.inf).max(axis=-1)
    m = np.where(ok, np.abs(ref), -np.inf).max(axis=-1)
    return np.where(ok.any(axis=-1), d / np.where(ok.any(axis=-1), m, 1.0), np.nan)


def check_rows(tag, y, ref):
    e = per_row(y, ref).reshape(-1)
    e = e[np.isfinite(e)]
    assert e.size > 0
    say(tag, "max", float(e.max()), "median", float(np.median(e)))
    assert np.all(np.isfinite(y))
    assert e.max() <= TOL_F and np.median(e) <= TOL_F_MEDIAN


# (layer, sub-layer, with inter-residual): the first and the last block, and
# the inter-residual point after block 2
DENSE_SUBS = [(0, 0, False), (0, 1, False), (3, 0, False), (3, 1, False), (1, 1, True)]


@pytest.mark.parametrize("layer,sub,inter", DENSE_SUBS)
def test_mxfp8_dense_sublayer_f_visible(layer, sub, inter):
    """Uneven mixing (H = 8): the Mix sub-layer at W = 512, Revert at 256."""
    require_gpu()
    import torch
    wl = visible(3)
    ctx, banks, ws = _ctx(3)
    say("MXFP8 F-visible dense sub-layer", wl.name, layer, sub, inter)
    x = dg.make_x(wl)
    xd = to_dev(wl, x)
    out = torch.empty_like(xd)
    rows = tile_rows(wl.B, 64, seed=100 + layer + sub)
    if sub == 0:
        ctx.sublayer_forward(layer, 0, xd, None, None, out, wl.B, stream())
        torch.cuda.synchronize()
        ref = oracle_sublayer(wl, ws, layer + 1, 0, x[rows].astype(np.float64))
    else:
        xr = dg.make_x(wl, seed=wl.seed + 100)
        ex = dg.make_x(wl, seed=wl.seed + 200) if inter else None
        ctx.sublayer_forward(layer, 1, to_dev(wl, xr), xd, to_dev(wl, ex) if inter else None, out, wl.B, stream())
        torch.cuda.synchronize()
        ref = oracle_sublayer(wl, ws, layer + 1, 1, xr[rows].astype(np.float64), x[rows].astype(np.float64),
                              ex[rows].astype(np.float64) if inter else None)
    check_rows(f"MXFP8 F-visible dense {layer} {sub} {inter}", to_np(out)[rows], ref)


def test_mxfp8_dense_revert_zero_residual_full_batch():
    require_gpu()
    import torch
    wl = visible(3)
    ctx, banks, ws = _ctx(3)
    x = dg.make_x(wl)
    xd = to_dev(wl, x)
    out = torch.empty_like(xd)
    ctx.sublayer_forward(0, 1, xd, torch.zeros_like(xd), None, out, wl.B, stream())
    torch.cuda.synchronize()
    rows = tile_rows(wl.B, 64, seed=130)
    ref = oracle_sublayer(wl, ws, 1, 1, x[rows].astype(np.float64), np.zeros((rows.size, wl.T, wl.D)))
    check_rows("MXFP8 F-visible dense F alone", to_np(out)[rows], ref)
    drop("mxfv3")


# the large MoE stack's oracle quantises every expert it evaluates (about
# 5 s per position on one core): a position from each end and two inside,
# on different XCDs' position ranges
MOE_POSITIONS = {4: None, 5: (0, 9, 22, 31)}


def _moe_check(ctx, wl, ws, layer, sub, xin, resid, extra, out, rows, tag, positions=None):
    idx_g, gate_g = route_gpu(ctx, wl, layer, sub, xin, wl.B)
    xr = to_np(xin)[rows]
    idx_o, gate_o, logits, bound = route_oracle(wl, ws, layer + 1, sub, xr)
    nb = check_routing(wl, idx_g[rows], gate_g[rows], idx_o, gate_o, logits, bound)
    ref = oracle_sublayer(wl, ws, layer + 1, sub, xr, None if resid is None else to_np(resid)[rows],
                          None if extra is None else to_np(extra)[rows], route=idx_g[rows], positions=positions)
    say(tag, "banded routes", nb)
    check_rows(tag, to_np(out)[rows], ref)


@pytest.mark.parametrize("wid", [4, 5])
def test_mxfp8_moe_sublayers_f_visible(wid):
    """Both sub-layers of the first and the last block, teacher-forced, plus
    the Revert sub-layer with a zero residual (F alone)."""
    require_gpu()
    import torch
    wl = visible(wid)
    say("MXFP8 F-visible MoE", wl.name, "(generating weights on first use)")
    ctx, banks, ws = _ctx(wid)
    x = to_dev(wl, dg.make_x(wl))
    x2 = to_dev(wl, dg.make_x(wl, seed=wl.seed + 100))
    rows = tile_rows(wl.B, 64, seed=140 + wid)
    pos = MOE_POSITIONS[wid]
    for layer in (0, wl.L - 1):
        out = torch.empty_like(x)
        ctx.sublayer_forward(layer, 0, x, None, None, out, wl.B, stream())
        torch.cuda.synchronize()
        _moe_check(ctx, wl, ws, layer, 0, x, None, None, out, rows,
                   f"MXFP8 F-visible MoE {wid} block {layer} mix", pos)
        ctx.sublayer_forward(layer, 1, x2, x, None, out, wl.B, stream())
        torch.cuda.synchronize()
        _moe_check(ctx, wl, ws, layer, 1, x2, x, None, out, rows,
                   f"MXFP8 F-visible MoE {wid} block {layer} revert", pos)
    zero = torch.zeros_like(x)
    out = torch.empty_like(x)
    ctx.sublayer_forward(0, 1, x2, zero, None, out, wl.B, stream())
    torch.cuda.synchronize()
    _moe_check(ctx, wl, ws, 0, 1, x2, zero, None, out, rows, f"MXFP8 F-visible MoE {wid} F alone", pos)
    drop(f"mxfv{wid}")

"""The F-visible GPU comparisons (tests/test_gpu_f_visible.py) can see F and
the Mix map: on the CPU, mistakes planted in the oracle -- F = 0 (every
down matrix zero, i.e. a kernel computing no FFN) and a plain-reshape Mix /
Revert (a kernel that forgot the permutation, reshaping [T, D] to
[H, T*D/H] without the transpose) -- move each compared quantity by at
least 10x the bf16 limit, on the same workloads (down_scale = 1) and the
same kinds of comparison: whole dense stacks, single sub-layers of both
kinds, and the Revert sub-layer with a zero residual. With the pages' own
down x 0.01 init the same mutations stay under the limit, which is why
those tests exist."""
import numpy as np
import pytest

import datagen as dg
import oracle as orc
import oracle.tmx_oracle as orc_mod

LIMIT = 2e-2
MARGIN = 10.0


def _row_err(y, ref):
    return float(np.max(np.max(np.abs(y - ref), -1) / np.max(np.abs(ref), -1)))


class _ZeroDown:
    def __init__(self, ws):
        self.ws = ws

    def __call__(self, layer, sub, kind, p):
        w = self.ws(layer, sub, kind, p)
        return np.zeros_like(w) if kind in dg.DOWN_KINDS else w


def _reshape_mix(X, H):
    B, T, D = X.shape
    return X.reshape(B, H, T * D // H)


def _reshape_revert(Hm, T):
    B, H, W = Hm.shape
    return Hm.reshape(B, T, H * W // T)


def _with_reshape_map(monkeypatch):
    monkeypatch.setattr(orc_mod, "mix", _reshape_mix)
    monkeypatch.setattr(orc_mod, "revert", _reshape_revert)


def _sublayer(wl, ws, sub, x, zero_resid=False):
    rho = True
    if sub == 0:
        Hm = orc_mod.mix(x, wl.H)
        return orc_mod.revert(orc_mod.sublayer_positions(Hm, Hm, wl, 1, 0, ws, None, rho), wl.T)
    resid = np.zeros_like(x) if zero_resid else dg.make_x(wl, seed=wl.seed + 7, B=x.shape[0]).astype(np.float64)
    return orc_mod.sublayer_positions(x, resid, wl, 1, 1, ws, None, rho)


def _vis(wid, **kw):
    wl = dg.WORKLOADS[wid]
    return wl.with_(name=wl.name + "_fvis", down_scale=1.0, **kw)


@pytest.mark.parametrize("wid", [2, 3])
def test_dense_stack_mutations_fail(wid, monkeypatch):
    wl = _vis(wid)
    ws = dg.WeightSource(wl, dg.weight_banks(wl))
    x = dg.make_x(wl, B=4).astype(np.float64)
    ref = orc.stack_forward(x, wl, ws)
    assert _row_err(orc.stack_forward(x, wl, _ZeroDown(ws)), ref) >= MARGIN * LIMIT
    with monkeypatch.context() as m:
        _with_reshape_map(m)
        assert _row_err(orc_mod.stack_forward(x, wl, ws), ref) >= MARGIN * LIMIT
    # the pages' init: the same mutation of F stays under the limit
    wl0 = dg.WORKLOADS[wid]
    ws0 = dg.WeightSource(wl0, dg.weight_banks(wl0))
    ref0 = orc.stack_forward(x, wl0, ws0)
    assert _row_err(orc.stack_forward(x, wl0, _ZeroDown(ws0)), ref0) < LIMIT


@pytest.mark.parametrize("wid", [2, 3, 4, 5])
@pytest.mark.parametrize("sub", [0, 1])
def test_sublayer_mutations_fail(wid, sub, monkeypatch):
    wl = _vis(wid, L=1)
    ws = dg.WeightSource(wl, dg.weight_banks(wl))
    x = dg.make_x(wl, B=4).astype(np.float64)
    ref = _sublayer(wl, ws, sub, x)
    assert _row_err(_sublayer(wl, _ZeroDown(ws), sub, x), ref) >= MARGIN * LIMIT
    if sub == 0:
        # the Mix sub-layer is where the map acts (the Revert sub-layer's map
        # is the identity)
        with monkeypatch.context() as m:
            _with_reshape_map(m)
            assert _row_err(_sublayer(wl, ws, sub, x), ref) >= MARGIN * LIMIT
    else:
        f_alone = _sublayer(wl, ws, 1, x, zero_resid=True)
        assert _row_err(_sublayer(wl, _ZeroDown(ws), 1, x, zero_resid=True), f_alone) >= MARGIN * LIMIT


# MXFP8 (tests/test_gpu_mxfp8_f_visible.py): rows are held to 2^-4 and the
# median row to 5e-3; the mutations must break both by 10x
MX_LIMIT, MX_MEDIAN = 2.0 ** -4, 5e-3


def _mx_sublayer(wl, ws, sub, x, zero_resid=False):
    # MoE: the first and the last position only (the oracle quantises every
    # expert it evaluates); the other positions' elements are NaN
    pos = (0, wl.positions(sub) - 1) if wl.moe else None
    if sub == 0:
        Hm = orc_mod.mix(x, wl.H)
        return orc_mod.revert(orc_mod.sublayer_positions(Hm, Hm, wl, 1, 0, ws, None, True, None, True,
                                                         positions=pos), wl.T)
    resid = np.zeros_like(x) if zero_resid else dg.make_x(wl, seed=wl.seed + 7, B=x.shape[0]).astype(np.float64)
    return orc_mod.sublayer_positions(x, resid, wl, 1, 1, ws, None, True, None, True, positions=pos)


def _row_errs(y, ref):
    """Row-normwise errors over the elements both sides evaluated."""
    ok = ~np.isnan(ref) & ~np.isnan(y)
    keep = ok.any(-1)
    d = np.where(ok, np.abs(y - ref), -np.inf).max(-1)[keep]
    m = np.where(ok, np.abs(ref), -np.inf).max(-1)[keep]
    return d / m


@pytest.mark.parametrize("wid", [3, 4])
@pytest.mark.parametrize("sub", [0, 1])
def test_mxfp8_sublayer_mutations_fail(wid, sub, monkeypatch):
    wl = _vis(wid, L=1, dtype="mxfp8")
    ws = dg.WeightSource(wl, dg.weight_banks(wl))
    x = dg.make_x(wl, B=4).astype(np.float64)

    def broken(e):
        return e.max() >= MARGIN * MX_LIMIT and np.median(e) >= MARGIN * MX_MEDIAN

    ref = _mx_sublayer(wl, ws, sub, x)
    assert broken(_row_errs(_mx_sublayer(wl, _ZeroDown(ws), sub, x), ref))
    if sub == 0:
        with monkeypatch.context() as m:
            _with_reshape_map(m)
            assert broken(_row_errs(_mx_sublayer(wl, ws, sub, x), ref))
    else:
        f_alone = _mx_sublayer(wl, ws, 1, x, zero_resid=True)
        assert broken(_row_errs(_mx_sublayer(wl, _ZeroDown(ws), 1, x, zero_resid=True), f_alone))

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


def oracle_sublayer(wl, ws, layer, sub, x_rows, resid_rows=None, extra_rows=None, route=None, positions=None):
    """Oracle of one sub-layer in block layout [n, T, D] (layer is 1-based);
    ``route`` [n, P, top_k] names the chosen experts of an MoE sub-layer
    (the other side's choice, once checked to be a correct one);
    ``positions`` evaluates only those positions of the sub-layer (the
    elements of the others are NaN)."""
    rho = wl.bf16_values
    mx = wl.dtype == "mxfp8"
    if sub == 0:
        Hm = orc.mix(x_rows, wl.H)
        return orc.revert(orc.sublayer_positions(Hm, Hm, wl, layer, 0, ws, None, rho, None, mx, route, positions),
                          wl.T)
    return orc.sublayer_positions(x_rows, resid_rows, wl, layer, 1, ws, extra_rows, rho, None, mx, route, positions)


def tile_rows(B, bm, seed=0):
    """One seeded row from every bm-row tile of the batch (every tile a
    persistent workgroup runs, its second and later tiles included)."""
    rng = np.random.default_rng(2000 + seed)
    starts = np.arange(0, B, bm)
    return np.minimum(starts + rng.integers(0, bm, starts.size), B - 1)


DELTA = {"bf16": 1e-3, "mxfp8": 1e-3, "f32": 1e-5}   # (MXFP8 routes on the bf16 x_hat, as bf16)


def route_gpu(ctx, wl, layer, sub, xd, B):
    import torch
    P = wl.positions(sub)
    idx = torch.empty((B, P, wl.top_k), dtype=torch.int32, device="cuda")
    gate = torch.empty((B, P, wl.top_k), dtype=torch.float32, device="cuda")
    ctx.moe_route(layer, sub, xd, B, idx, gate, stream())
    torch.cuda.synchronize()
    return idx.cpu().numpy(), gate.cpu().numpy().astype(np.float64)


def norm_near_midpoint(z, W):
    """Elements of the normalised rows z (fp64) whose bf16 rounding the GPU may
    take the other way, and their ulps. The kernel forms z in fp32: the sum of
    squares is a chain of at most W/4 products and additions per lane plus a
    4-lane butterfly, then the mean, eps, square root, reciprocal and two
    products, so |z_fp32 - z| <= (W/4 + 8) 2^-24 |z|, which is at most
    (W/4 + 8) 2^-16 of a bf16 ulp of z. An element rounds alike on both sides
    unless z lies that close to a rounding midpoint."""
    _, ex = np.frexp(z)
    ulp = np.ldexp(1.0, ex - 8)
    frac = z / ulp - np.floor(z / ulp)
    return np.abs(frac - 0.5) <= (W / 4 + 8) * 2.0 ** -16, ulp


def logit_acc_bound(xh, wr):
    """Per row, a bound on the fp32 accumulation error of the router's
    logits: each is accumulated over W/32 MFMA steps of 32 products, every
    step adding at most a few roundings, so |d logit_e| <= (W/32 + 8) 2^-24
    sum_i |x_i w_ie|. Large logits (a dominant router column) carry errors
    of several 1e-6 absolute, which is the gate's relative error."""
    W = xh.shape[-1]
    return (W / 32 + 8) * 2.0 ** -24 * np.max(np.abs(xh) @ np.abs(wr), axis=-1)


def route_oracle(wl, ws, layer1, sub, x_rows):
    """Oracle routing of rows x_rows [n, T, D] (block layout).

    Also returns, per (row, position), a bound on how far the GPU's logits
    can lie from the oracle's: an element of x_hat near a bf16 rounding
    midpoint (norm_near_midpoint) may round either way, changing logit e by
    at most ulp_i * |Wr[i, e]|, and the GPU accumulates in fp32
    (logit_acc_bound)."""
    rho = wl.bf16_values
    v = orc.mix(x_rows, wl.H) if sub == 0 else x_rows
    n, P, W = v.shape
    out, bound = [], []
    for p in range(P):
        z = orc.rmsnorm(v[:, p], ws(layer1, sub, dg.K_NORM_GAIN, 0), wl.eps)
        wr = ws(layer1, sub, dg.K_ROUTER, p).astype(np.float64)
        if rho:
            near, ulp = norm_near_midpoint(z, W)
            xh = orc.round_bf16(z)
            bound.append(np.max((near * ulp) @ np.abs(wr), axis=-1) + logit_acc_bound(xh, wr))
        else:
            bound.append(np.zeros(n))
            xh = z
        out.append(orc.route(xh, wr, wl.top_k, wl.gate_scale))
    idx = np.stack([o[0] for o in out], 1)
    gate = np.stack([o[1] for o in out], 1)
    logits = np.stack([o[2] for o in out], 1)
    return idx, gate, logits, np.stack(bound, 1)


def check_routing(wl, idx_g, gate_g, idx_o, gate_o, logits, bound):
    """Per (row, position) band d = max(delta, 2.05 * bound): indices must be
    exact where the k-th/(k+1)-th logit margin exceeds d (each logit can move
    by at most `bound`, plus fp32 accumulation slack inside delta); the other
    rows must be d-valid. Gates within 1e-5 relative plus the effect of the
    x_hat rounding bound (softmax: |d log pi| <= 2 max |d logit|).
    Returns the number of banded rows."""
    k, E = wl.top_k, logits.shape[-1]
    dband = np.maximum(DELTA[wl.dtype], 2.05 * bound)
    srt = -np.sort(-logits, axis=-1)
    kth = srt[..., k - 1]
    margin = kth - (srt[..., k] if k < E else -np.inf)
    clear = margin > dband
    assert np.array_equal(idx_g[clear], idx_o[clear])
    rtol = 1e-5 + 2.1 * bound
    # fp32 gates below the normal range (2^-126) keep only the absolute
    # spacing 2^-149; the gate alpha * exp(l - m) / den is within one such
    # spacing of its rounding, scaled by alpha
    atol = wl.gate_scale * 2.0 ** -148
    dev = np.abs(gate_g - gate_o) - atol
    rel = np.maximum(dev, 0.0) / np.abs(gate_o)
    bad = np.argwhere(clear[..., None] & (rel > rtol[..., None]))
    for pos in bad[np.argsort(-rel[tuple(bad.T)])][:8]:
        r = tuple(pos[:-1])
        print("[gate mismatch] row/pos", r, "slot", pos[-1], "expert", idx_g[r][pos[-1]], "gpu", gate_g[tuple(pos)],
              "oracle", gate_o[tuple(pos)], "bound", bound[r], "logits", np.round(logits[r], 5).tolist(), flush=True)
    assert bad.shape[0] == 0, (int(bad.shape[0]), float(np.max(rel[tuple(bad.T)])))
    band = np.argwhere(~clear)
    for pos in band:
        r = tuple(pos)
        d = dband[r]
        chosen = set(idx_g[r].tolist())
        assert len(chosen) == k
        l = logits[r]
        for e in range(E):
            if e in chosen:
                assert l[e] >= kth[r] - d
            else:
                assert l[e] <= kth[r] + d
    return len(band)





def check_xhat_and_route(wl, ws, layer1, sub, x_rows, xhat_rows, idx_g, gate_g):
    """The GPU's normalised rows and its routing, each against what it must be.

    x_hat: every element is rho(z) of the fp64 RMSNorm z, except elements near
    a rounding midpoint (norm_near_midpoint), which may be the other
    neighbour. Routing: computed in fp64 from the GPU's own x_hat, the logits
    differ from the GPU's fp32 ones only by accumulation error
    (logit_acc_bound). Indices must be equal where the k-th / (k+1)-th
    margin exceeds twice the row's largest such bound; elsewhere the choice
    must be valid within it. Gates: the GPU's log gate moves by at most
    4 max |d logit| plus the roundings of the fp32 difference to the largest
    logit, the exponential, the division and the scale, plus the absolute
    spacing of fp32 below its normal range. x_rows [n, T, D] block layout, xhat_rows [n, P, W].
    Returns (x_hat elements taking the other neighbour, banded rows)."""
    u = 2.0 ** -24
    v = orc.mix(x_rows, wl.H) if sub == 0 else x_rows
    n, P, W = v.shape
    k, E = wl.top_k, wl.E
    flips, banded = 0, 0
    for p in range(P):
        z = orc.rmsnorm(v[:, p], ws(layer1, sub, dg.K_NORM_GAIN, 0), wl.eps)
        xh = xhat_rows[:, p].astype(np.float64)
        rz = orc.round_bf16(z)
        diff = xh != rz
        near, ulp = norm_near_midpoint(z, W)
        assert np.all(near[diff]), int(np.sum(diff & ~near))
        assert np.all(np.abs(xh - z)[diff] <= ulp[diff])
        flips += int(np.sum(diff))
        wr = ws(layer1, sub, dg.K_ROUTER, p).astype(np.float64)
        idx_o, gate_o, logits, _ = orc.route(xh, wr, k, wl.gate_scale)
        dl = logit_acc_bound(xh, wr)                                # per row
        srt = -np.sort(-logits, axis=-1)
        kth = srt[:, k - 1]
        margin = kth - (srt[:, k] if k < E else -np.inf)
        clear = margin > 2 * dl
        ig = idx_g[:, p]
        assert np.array_equal(ig[clear], idx_o[clear])
        for r in np.nonzero(~clear)[0]:
            chosen = set(ig[r].tolist())
            assert len(chosen) == k and all(0 <= e < E for e in chosen)
            for e in range(E):
                if e in chosen:
                    assert logits[r, e] >= kth[r] - 2 * dl[r]
                else:
                    assert logits[r, e] <= kth[r] + 2 * dl[r]
        banded += int(np.sum(~clear))
        sel = ig.astype(np.int64)
        go = wl.gate_scale * np.take_along_axis(orc.softmax(logits), sel, axis=-1)
        gg = gate_g[:, p]
        # logit_e - max and log(den) each move by at most 2 dl; the fp32
        # difference logit_e - max is rounded (u |logit_e - max| absolute);
        # exp, the division and the scale add a few u
        gap = np.max(logits, axis=-1, keepdims=True) - np.take_along_axis(logits, sel, axis=-1)
        rtol = 4 * dl[:, None] + u * (gap + 16)
        atol = wl.gate_scale * 2.0 ** -148
        assert np.all(np.abs(gg - go) <= rtol * np.abs(go) + atol), float(np.max(np.abs(gg - go) / np.abs(go)))
    return flips, banded

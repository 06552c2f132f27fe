"""Sparse-Pertoken MoE path on the GPU (router, bucket, grouped experts,
shared expert + combine) vs the fp64 oracle."""
import numpy as np
import pytest

import datagen as dg
import oracle as orc
from gpu_common import (TOL, check_routing, check_xhat_and_route, context, drop, oracle_sublayer, require_gpu,
                        route_gpu, route_oracle, row_err, sample_rows, say, stream, to_dev, to_np)

pytestmark = pytest.mark.gpu

# small MoE stack: ragged batch, W = 128 in both sub-layers
SMALL_MOE = dg.Workload("small_moe_bf16", B=300, T=4, H=4, D=128, L=3, E=16, top_k=4,
                        expert_hidden=128, shared_hidden=256, alpha=4.0, gap=2, seed=31)
SMALL_MOE_F32 = SMALL_MOE.with_(name="small_moe_f32", dtype="f32", B=64, D=32, E=6, top_k=2,
                                expert_hidden=16, shared_hidden=24, alpha=3.0, seed=32)
# wider expert sets: the router's logits span 3 and 4 MFMA column blocks, and
# the bucket kernel's per-expert tables reach their 64-expert limit
SMALL_MOE_E48 = SMALL_MOE.with_(name="small_moe_e48", E=48, top_k=6, alpha=8.0, seed=33)
SMALL_MOE_E64 = SMALL_MOE.with_(name="small_moe_e64", E=64, top_k=8, alpha=8.0, seed=34)
SMALL = {"small_bf16": SMALL_MOE, "small_f32": SMALL_MOE_F32, "small_e48": SMALL_MOE_E48,
         "small_e64": SMALL_MOE_E64}

@pytest.mark.parametrize("which", ["small_bf16", "small_f32", "small_e48", "small_e64"])
def test_small_moe_stack_all_rows(which):
    require_gpu()
    wl = SMALL[which]
    say("small moe stack", wl)
    ctx, banks, ws = context(which, wl)
    import torch
    x = dg.make_x(wl)
    xd = to_dev(wl, x)
    y = torch.empty_like(xd)
    ctx.block_stack_forward(xd, y, wl.B, stream())
    torch.cuda.synchronize()
    ref = orc.stack_forward(x.astype(np.float64), wl, ws)
    err = row_err(to_np(y), ref)
    say("small moe err", which, err)
    assert err <= TOL[wl.dtype]
    y2 = torch.empty_like(xd)
    ctx.block_stack_forward(xd, y2, wl.B, stream())
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


@pytest.mark.parametrize("which", ["small_bf16", "small_f32", "small_e48", "small_e64", "w4"])
@pytest.mark.parametrize("sub", [0, 1])
def test_route_matches_oracle(which, sub):
    require_gpu()
    wl = SMALL[which] if which in SMALL else dg.WORKLOADS[4]
    say("route", which, sub)
    ctx, banks, ws = context(which, wl)
    x = dg.make_x(wl)
    idx_g, gate_g = route_gpu(ctx, wl, 0, sub, to_dev(wl, x), wl.B)
    rows = sample_rows(wl.B, 512, seed=sub) if wl.B > 512 else np.arange(wl.B)
    idx_o, gate_o, logits, bound = route_oracle(wl, ws, 1, sub, x[rows].astype(np.float64))
    nb = check_routing(wl, idx_g[rows], gate_g[rows], idx_o, gate_o, logits, bound)
    say("route strict-gate rows", which, sub, int(np.sum(bound == 0)), "max bound", float(bound.max()))
    say("route banded rows", which, sub, nb, "of", idx_o.shape[0] * idx_o.shape[1])
    # every row's selection is k distinct experts
    s = np.sort(idx_g, axis=-1)
    assert np.all(s[..., 1:] != s[..., :-1]) and s.min() >= 0 and s.max() < wl.E
    if wl.dtype == "bf16":
        xhat = xhat_gpu(ctx, wl, 0, sub, to_dev(wl, x), wl.B)
        flips, nb2 = check_xhat_and_route(wl, ws, 1, sub, x[rows].astype(np.float64), xhat[rows],
                                          idx_g[rows], gate_g[rows])
        say("route from the GPU's x_hat", which, sub, "x_hat elements on the other neighbour", flips,
            "banded rows", nb2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_route_exact_ties_lowest_index(dtype):
    """Dyadic router weights, +-1 inputs and duplicated router columns: every
    logit is exact, ties are exact, and the lowest index must win."""
    require_gpu()
    import torch
    from token_moe_amd import runner
    wl = SMALL_MOE.with_(name="ties", L=1, B=256) if dtype == "bf16" else SMALL_MOE_F32.with_(name="ties32", L=1)
    banks = dg.weight_banks(wl)
    rng = np.random.default_rng(5)
    for sub in (0, 1):
        P, W, E = wl.positions(sub), wl.width(sub), wl.E
        half = rng.integers(-64, 65, (P, W, E // 2)).astype(np.float32) / np.float32(64.0)
        wr = np.concatenate([half, half], axis=-1)           # expert e and e + E/2 tie exactly
        banks[(1, sub, dg.K_ROUTER)] = dg.f32_to_bf16_bits(wr) if dtype == "bf16" else wr
    ctx = runner.make_context(wl, banks)
    ws = dg.WeightSource(wl, banks)
    x = np.where(rng.random((wl.B, wl.T, wl.D)) < 0.5, -1.0, 1.0).astype(np.float32)
    for sub in (0, 1):
        idx_g, gate_g = route_gpu(ctx, wl, 0, sub, to_dev(wl, x), wl.B)
        idx_o, gate_o, logits, _ = route_oracle(wl, ws, 1, sub, x.astype(np.float64))
        if dtype == "bf16":
            # x_hat = +-1 exactly, logits are exact dyadic sums: routing must match bit for bit
            np.testing.assert_array_equal(idx_g, idx_o)
        else:
            # fp32 x_hat = +-(1+eps)^-1/2 is inexact, but tied columns stay tied
            half = wl.E // 2
            lo = idx_g % half
            for r in np.ndindex(idx_g.shape[:2]):
                for s in range(wl.top_k):
                    e = idx_g[r][s]
                    if e >= half:   # an upper copy may only be taken after its lower twin
                        assert e - half in idx_g[r][:s].tolist()
        np.testing.assert_allclose(gate_g, gate_o, rtol=1e-5)
    ctx.close()


def buckets_gpu(ctx, wl, layer, sub, xd, B):
    import torch
    P = wl.positions(sub)
    counts = torch.empty((P, wl.E), dtype=torch.int32, device="cuda")
    rows = torch.empty((P, B * wl.top_k), dtype=torch.int32, device="cuda")
    ctx.moe_buckets(layer, sub, xd, B, None, counts, rows, stream())
    torch.cuda.synchronize()
    return counts.cpu().numpy(), rows.cpu().numpy()


def xhat_gpu(ctx, wl, layer, sub, xd, B):
    """The normalised rows the sub-layer's experts consume, [B, P, W]."""
    import torch
    P, W = wl.positions(sub), wl.width(sub)
    xh = torch.empty((P, B, W), dtype=torch.bfloat16, device="cuda")
    ctx.moe_buckets(layer, sub, xd, B, xh, None, None, stream())
    torch.cuda.synchronize()
    return to_np(xh).transpose(1, 0, 2)


def check_buckets(idx, counts, rows, E):
    """MoEPermute lists against the routing table: per position, expert e's
    count is the number of (row, slot) entries routed to it, its list starts
    at the exclusive prefix sum of the counts, and holds exactly those
    entries b * top_k + slot in ascending order (stable). Bit-exact."""
    B, P, k = idx.shape
    for p in range(P):
        flat = idx[:, p, :].reshape(-1)
        want = np.bincount(flat, minlength=E)
        np.testing.assert_array_equal(counts[p], want)
        off = np.concatenate([[0], np.cumsum(want)])
        for e in range(E):
            np.testing.assert_array_equal(rows[p, off[e]:off[e + 1]], np.nonzero(flat == e)[0])
        assert off[E] == B * k


@pytest.mark.parametrize("which", ["small_bf16", "w4"])
@pytest.mark.parametrize("sub", [0, 1])
def test_buckets_match_routing(which, sub):
    require_gpu()
    wl = {"small_bf16": SMALL_MOE, "w4": dg.WORKLOADS[4]}[which]
    say("buckets", which, sub)
    ctx, banks, ws = context(which, wl)
    xd = to_dev(wl, dg.make_x(wl))
    idx_g, _ = route_gpu(ctx, wl, 0, sub, xd, wl.B)
    counts, rows = buckets_gpu(ctx, wl, 0, sub, xd, wl.B)
    check_buckets(idx_g, counts, rows, wl.E)
    # a smaller batch through the same context: lists of the first rows only
    B2 = wl.B // 3 + 1
    idx2, _ = route_gpu(ctx, wl, 0, sub, xd[:B2].contiguous(), B2)
    c2, r2 = buckets_gpu(ctx, wl, 0, sub, xd[:B2].contiguous(), B2)
    np.testing.assert_array_equal(idx2, idx_g[:B2])
    check_buckets(idx2, c2, r2, wl.E)


@pytest.mark.parametrize("width", [128, 512])
@pytest.mark.parametrize("sub", [0, 1])
def test_skewed_routing_and_empty_buckets(sub, width):
    """Positive inputs, positive router columns except expert 5 (all
    negative): expert 5's bucket is always empty, and expert 3 (column x10)
    is chosen by every row, so its bucket holds all B rows (8 tiles of the
    128-row kernels: the fused one at W = 128, the wide routed-expert kernel
    at W = 512 with expert hidden 256). The
    down matrices at full scale and, in the Revert sub-layer, a zero
    residual make the sub-layer output F itself, so the all-rows bucket's
    expert outputs are what the comparison sees."""
    require_gpu()
    import torch
    from token_moe_amd import runner
    wl = SMALL_MOE.with_(name="skew", L=1, B=1000, down_scale=1.0)
    if width == 512:
        wl = wl.with_(name="skew512", D=512, expert_hidden=256, shared_hidden=512)
    banks = dg.weight_banks(wl)
    for s in (0, 1):
        wr = np.abs(dg.bf16_bits_to_f32(banks[(1, s, dg.K_ROUTER)]))
        wr[..., 3] *= 10.0
        wr[..., 5] = -wr[..., 5]
        banks[(1, s, dg.K_ROUTER)] = dg.f32_to_bf16_bits(wr)
    ctx = runner.make_context(wl, banks)
    ws = dg.WeightSource(wl, banks)
    x = np.abs(dg.make_x(wl))
    xd = to_dev(wl, x)
    idx_g, gate_g = route_gpu(ctx, wl, 0, sub, xd, wl.B)
    assert not np.any(idx_g == 5)
    assert np.all(idx_g[..., 0] == 3)
    counts, rows = buckets_gpu(ctx, wl, 0, sub, xd, wl.B)
    check_buckets(idx_g, counts, rows, wl.E)
    assert np.all(counts[:, 5] == 0) and np.all(counts[:, 3] == wl.B)
    out = torch.empty_like(xd)
    zero = np.zeros(x.shape)
    if sub == 0:
        ctx.sublayer_forward(0, 0, xd, None, None, out, wl.B, stream())
    else:
        ctx.sublayer_forward(0, 1, xd, torch.zeros_like(xd), None, out, wl.B, stream())
    torch.cuda.synchronize()
    flips, nb = check_xhat_and_route(wl, ws, 1, sub, x.astype(np.float64), xhat_gpu(ctx, wl, 0, sub, xd, wl.B),
                                     idx_g, gate_g)
    say("skew: x_hat elements on the other neighbour", flips, "banded", nb)
    idx_o, gate_o, logits, bound = route_oracle(wl, ws, 1, sub, x.astype(np.float64))
    check_routing(wl, idx_g, gate_g, idx_o, gate_o, logits, bound)
    ref = oracle_sublayer(wl, ws, 1, sub, x.astype(np.float64), None if sub == 0 else zero, route=idx_g)
    err = row_err(to_np(out), ref)
    say("skewed err", sub, err)
    assert err <= TOL["bf16"]
    ctx.close()


@pytest.mark.parametrize("sub", [0, 1])
def test_non_finite_row_keeps_routing_in_range(sub):
    """A row of +inf inputs makes its normalised row NaN. Its routing must
    still name top_k distinct experts in [0, E) (every bucket entry stays in
    range), and every other row's routing and buckets are those of the same
    batch without it."""
    require_gpu()
    import torch
    wl = SMALL_MOE
    ctx, banks, ws = context("small_bf16", wl)
    x = dg.make_x(wl)
    bad = 17
    xb = x.copy()
    xb[bad] = np.inf
    xd, xbd = to_dev(wl, x), to_dev(wl, xb)
    idx_ok, gate_ok = route_gpu(ctx, wl, 0, sub, xd, wl.B)
    idx_b, gate_b = route_gpu(ctx, wl, 0, sub, xbd, wl.B)
    s = np.sort(idx_b[bad], axis=-1)
    assert s.min() >= 0 and s.max() < wl.E and np.all(s[:, 1:] != s[:, :-1])
    keep = np.arange(wl.B) != bad
    np.testing.assert_array_equal(idx_b[keep], idx_ok[keep])
    np.testing.assert_array_equal(gate_b[keep], gate_ok[keep])
    counts, rows = buckets_gpu(ctx, wl, 0, sub, xbd, wl.B)
    check_buckets(idx_b, counts, rows, wl.E)
    out = torch.empty_like(xd)
    if sub == 0:
        ctx.sublayer_forward(0, 0, xbd, None, None, out, wl.B, stream())
    else:
        ctx.sublayer_forward(0, 1, xbd, xd, None, out, wl.B, stream())
    torch.cuda.synchronize()
    y = to_np(out)
    ref = oracle_sublayer(wl, ws, 1, sub, x[keep].astype(np.float64),
                          None if sub == 0 else x[keep].astype(np.float64), route=idx_b[keep])
    err = row_err(y[keep], ref)
    say("non-finite row: other rows err", sub, err)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("sub", [0, 1])
def test_moe_sublayer_teacher_forced_full_batch(sub):
    require_gpu()
    import torch
    wl = dg.WORKLOADS[4]
    say("moe sublayer cfg4", sub)
    ctx, banks, ws = context("w4", wl)
    x = dg.make_x(wl)
    xd = to_dev(wl, x)
    out = torch.empty_like(xd)
    rows = sample_rows(wl.B, 24, seed=40 + sub)
    if sub == 0:
        ctx.sublayer_forward(0, 0, xd, None, None, out, wl.B, stream())
        torch.cuda.synchronize()
        ref = oracle_sublayer(wl, ws, 1, 0, x[rows].astype(np.float64))
    else:
        xr = to_dev(wl, dg.make_x(wl, seed=wl.seed + 100))
        ctx.sublayer_forward(0, 1, xr, xd, None, out, wl.B, stream())
        torch.cuda.synchronize()
        ref = oracle_sublayer(wl, ws, 1, 1, to_np(xr)[rows], x[rows].astype(np.float64))
    err = row_err(to_np(out)[rows], ref)
    say("moe sublayer err", sub, err)
    assert err <= TOL["bf16"]


def test_moe_stack_full_batch_sampled():
    require_gpu()
    import torch
    wl = dg.WORKLOADS[4]
    say("moe stack cfg4")
    ctx, banks, ws = context("w4", wl)
    x = dg.make_x(wl)
    xd = to_dev(wl, x)
    y = torch.empty_like(xd)
    ctx.block_stack_forward(xd, y, wl.B, stream())
    torch.cuda.synchronize()
    rows = sample_rows(wl.B, 8, seed=44)
    ref = orc.stack_forward(x[rows].astype(np.float64), wl, ws)
    err = row_err(to_np(y)[rows], ref)
    say("moe stack err", err)
    assert err <= TOL["bf16"]
    drop("w4")


# ---------------------------------------------------------------------------
# the large MoE stack (B=8192, T=H=32, D=768, E=32, ~15.4e9 weights) at full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("sub", [0, 1])
def test_large_moe_sublayer_and_route_full_batch(sub):
    require_gpu()
    import torch
    wl = dg.WORKLOADS[5]
    say("large moe: generating / uploading weights (first use)", sub)
    ctx, banks, ws = context("w5", wl)
    x = dg.make_x(wl)
    xd = to_dev(wl, x)
    # routing of sampled rows, teacher-forced on the same input
    idx_g, gate_g = route_gpu(ctx, wl, 0, sub, xd, wl.B)
    rows = sample_rows(wl.B, 192, seed=50 + sub)
    idx_o, gate_o, logits, bound = route_oracle(wl, ws, 1, sub, x[rows].astype(np.float64))
    nb = check_routing(wl, idx_g[rows], gate_g[rows], idx_o, gate_o, logits, bound)
    say("large route banded rows", sub, nb)
    xhat = xhat_gpu(ctx, wl, 0, sub, xd, wl.B)
    flips, nb2 = check_xhat_and_route(wl, ws, 1, sub, x[rows].astype(np.float64), xhat[rows], idx_g[rows],
                                      gate_g[rows])
    say("large route from the GPU's x_hat: other-neighbour elements", flips, "banded", nb2)
    # one sub-layer at the full batch, oracle on sampled rows
    out = torch.empty_like(xd)
    rows = sample_rows(wl.B, 10, seed=60 + sub)
    if sub == 0:
        ctx.sublayer_forward(0, 0, xd, None, None, out, wl.B, stream())
        torch.cuda.synchronize()
        ref = oracle_sublayer(wl, ws, 1, 0, x[rows].astype(np.float64))
    else:
        xr = to_dev(wl, dg.make_x(wl, seed=wl.seed + 100))
        ctx.sublayer_forward(0, 1, xr, xd, None, out, wl.B, stream())
        torch.cuda.synchronize()
        ref = oracle_sublayer(wl, ws, 1, 1, to_np(xr)[rows], x[rows].astype(np.float64))
    err = row_err(to_np(out)[rows], ref)
    say("large moe sublayer err", sub, err)
    assert err <= TOL["bf16"]


def test_large_moe_stack_full_batch_sampled():
    require_gpu()
    import torch
    wl = dg.WORKLOADS[5]
    ctx, banks, ws = context("w5", wl)
    x = dg.make_x(wl)
    xd = to_dev(wl, x)
    y = torch.empty_like(xd)
    ctx.block_stack_forward(xd, y, wl.B, stream())
    torch.cuda.synchronize()
    yn = to_np(y)
    assert np.all(np.isfinite(yn[::97]))
    rows = sample_rows(wl.B, 3, seed=70)
    ref = orc.stack_forward(x[rows].astype(np.float64), wl, ws)
    err = row_err(yn[rows], ref)
    say("large moe stack err", err)
    assert err <= TOL["bf16"]
    drop("w5")

"""Stacks with MXFP8 GEMM operands (TMX_MXFP8) on the GPU vs the oracle's
MXFP8 reading of the FP8 serving path (TokenMixer-Large 2.5.2): dense
sub-layers at W = 256 and 512, MoE sub-layers (routed and shared experts) at
W = 512.

Tolerances. The kernel and the oracle quantise the same quantities, but
from fp32 values that differ in their last bits (fp32 norm statistics and
accumulation against fp64). A value near a rounding boundary can take the
neighbouring E4M3 code, and a block whose maximum sits at a power of two can
take the neighbouring shared exponent, which requantises its 32 values. Each
value then moves by at most half a step of the coarser grid, 2^-4 of itself,
so the SwiGLU output F of a row is within 2^-4 (row-normwise) of the
oracle's. Rows where the residual dominates stay within the bf16 bound
(2e-2). F alone is checked with a zero residual, against 2^-4 for the worst
row and 5e-3 for the median row: a layout or scale error moves every row,
not a few."""
import numpy as np
import pytest

import datagen as dg
import oracle as orc
from gpu_common import (TOL, check_routing, context, drop, oracle_sublayer, require_gpu, route_gpu, route_oracle,
                        row_err, sample_rows, say, stream, to_dev, to_np)

pytestmark = pytest.mark.gpu

# W = 256 in both sub-layers (P = 16), ragged batch (1000 = 15 * 64 + 40),
# 2 and 3 hidden chunks, inter-residual at block 2
TOL_F = 2.0 ** -4          # F alone, worst row
TOL_F_MEDIAN = 5e-3        # F alone, median row

MX_SMALL = dg.Workload("mx_small_dense", B=1000, T=16, H=16, D=256, L=3, hidden_mix=256,
                       hidden_rev=384, gap=2, dtype="mxfp8", seed=41)


def _stack(ctx, x_dev, B):
    import torch
    y = torch.empty_like(x_dev)
    ctx.block_stack_forward(x_dev, y, B, stream())
    torch.cuda.synchronize()
    return y


def test_mxfp8_small_stack_all_rows():
    require_gpu()
    wl = MX_SMALL
    say("mxfp8 small stack", wl)
    ctx, banks, ws = context("mx_small", wl)
    x = dg.make_x(wl)
    y = to_np(_stack(ctx, to_dev(wl, x), wl.B))
    ref = orc.stack_forward(x.astype(np.float64), wl, ws)
    err = row_err(y, ref)
    say("mxfp8 small err", err)
    assert err <= TOL["bf16"]
    assert np.all(np.isfinite(y))
    # the quantisation is real: the bf16-path oracle differs by more than the parity error
    ref_bf16 = orc.stack_forward(x.astype(np.float64), wl, ws, rho=True, mx=False)
    dev = row_err(y, ref_bf16)
    say("mxfp8 vs bf16 path", dev)
    assert dev > err and dev < 0.1


@pytest.mark.parametrize("sub", [0, 1])
def test_mxfp8_sublayer_teacher_forced_full_batch(sub):
    """One sub-layer at the dense stack's full batch (B = 4096, T = H = 16,
    D = 256, hidden 1024), sampled rows."""
    require_gpu()
    import torch
    wl = dg.WORKLOADS[2].with_(name="mx_dense_pertoken", dtype="mxfp8", L=1)
    say("mxfp8 sublayer", sub)
    ctx, banks, ws = context("mx_w2", wl)
    x = dg.make_x(wl)
    xd = to_dev(wl, x)
    out = torch.empty_like(xd)
    if sub == 0:
        ctx.sublayer_forward(0, 0, xd, None, None, out, wl.B, stream())
    else:
        ctx.sublayer_forward(0, 1, xd, xd, None, out, wl.B, stream())
    torch.cuda.synchronize()
    rows = sample_rows(wl.B, 32, seed=sub)
    xr = x[rows].astype(np.float64)
    ref = oracle_sublayer(wl, ws, 1, sub, xr, xr if sub == 1 else None)
    err = row_err(to_np(out)[rows], ref)
    say("mxfp8 sublayer err", sub, err)
    assert err <= TOL["bf16"]


def test_mxfp8_deterministic_and_unsupported_shapes():
    require_gpu()
    import torch
    from token_moe_amd import runner, tmx
    wl = MX_SMALL
    ctx, banks, ws = context("mx_small", wl)
    xd = to_dev(wl, dg.make_x(wl))
    assert torch.equal(_stack(ctx, xd, wl.B), _stack(ctx, xd, wl.B))
    # W = 768; MoE at W = 256; a hidden past 8 chunks
    for bad in (dict(D=768), dict(E=16, top_k=4, expert_hidden=256, shared_hidden=512), dict(hidden_mix=2048)):
        cfg = runner.config_from_workload(wl.with_(**bad))
        with pytest.raises(tmx.TmxError) as e:
            tmx.Context(cfg)
        assert e.value.status == tmx.TMX_ERR_UNSUPPORTED


def test_mxfp8_zero_and_scaled_rows_and_batch_independence():
    """Rows of zeros (block maximum 0: the smallest scale), rows scaled by
    2^12 and 2^-12 (other block exponents, same codes), and B = 1 / ragged
    calls giving the same rows bit for bit."""
    require_gpu()
    import torch
    wl = MX_SMALL.with_(name="mx_edges", B=200, L=1, seed=43)
    ctx, banks, ws = context("mx_edges", wl)
    x = dg.make_x(wl).copy()
    x[3] = 0.0
    x[5] *= np.float32(2.0 ** 12)
    x[7] *= np.float32(2.0 ** -12)
    x = dg.to_bf16_values(x)
    xd = to_dev(wl, x)
    y = _stack(ctx, xd, wl.B)
    ref = orc.stack_forward(x.astype(np.float64), wl, ws)
    yn = to_np(y)
    assert np.all(np.isfinite(yn))
    assert np.array_equal(yn[3], ref[3])          # zero row: zero input, zero hidden, zero output
    # sample 7 is scaled so far down that eps dominates its norm: its
    # residual is as small as F, so it is held to the F bound; the others
    # (the 2^12-scaled sample 5 included) to the bf16 bound
    rows = [r for r in range(wl.B) if r not in (3, 7)]
    err = row_err(yn[rows], ref[rows])
    err7 = row_err(yn[7], ref[7])
    say("mxfp8 edge rows err", err, "eps-dominated sample", err7)
    assert err <= TOL["bf16"] and err7 <= TOL_F
    for B in (1, 129):
        yb = _stack(ctx, xd[:B].contiguous(), B)
        assert torch.equal(yb, y[:B])


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8"])
def test_swiglu_alone_zero_residual(dtype):
    """The Revert sub-layer with a zero residual returns F(RMSNorm(x)) alone,
    so the comparison is not dominated by the residual: bf16 within the bf16
    bound, MXFP8 within the F bounds above."""
    require_gpu()
    import torch
    wl = dg.Workload("f_only_" + dtype, B=256, T=16, H=16, D=256, L=1, hidden_mix=256, hidden_rev=384,
                     gap=0, dtype=dtype, seed=51)
    ctx, banks, ws = context("f_only_" + dtype, wl)
    x = dg.make_x(wl)
    xd = to_dev(wl, x)
    out = torch.empty_like(xd)
    ctx.sublayer_forward(0, 1, xd, torch.zeros_like(xd), None, out, wl.B, stream())
    torch.cuda.synchronize()
    ref = oracle_sublayer(wl, ws, 1, 1, x.astype(np.float64), np.zeros(x.shape))
    y = to_np(out)
    per_row = np.max(np.abs(y - ref), axis=-1) / np.max(np.abs(ref), axis=-1)
    say("F alone", dtype, "max", per_row.max(), "median", np.median(per_row))
    if dtype == "bf16":
        assert per_row.max() <= TOL["bf16"]
    else:
        assert per_row.max() <= TOL_F and np.median(per_row) <= TOL_F_MEDIAN


# ---------------------------------------------------------------------------
# W = 512: dense (Mix of H = 8) and MoE sub-layers
# ---------------------------------------------------------------------------

# Mix W = 512 (T = 16, H = 8, D = 256), Revert W = 256; 3 and 2 hidden
# chunks; ragged batch (1000 = 15 * 64 + 40)
MX_DENSE_512 = dg.Workload("mx_dense_512", B=1000, T=16, H=8, D=256, L=2, hidden_mix=384,
                           hidden_rev=256, gap=2, dtype="mxfp8", seed=45)
# MoE at W = 512 in both sub-layers (T = H = 4, D = 512): 2 chunks per
# routed expert, 3 for the shared one; ragged batch
MX_MOE_SMALL = dg.Workload("mx_moe_small", B=300, T=4, H=4, D=512, L=2, E=16, top_k=4,
                           expert_hidden=256, shared_hidden=384, alpha=4.0, gap=2, dtype="mxfp8", seed=46)


@pytest.mark.parametrize("which", ["dense_512", "moe_small"])
def test_mxfp8_w512_small_stack_all_rows(which):
    require_gpu()
    wl = MX_DENSE_512 if which == "dense_512" else MX_MOE_SMALL
    say("mxfp8 W=512 stack", wl)
    ctx, banks, ws = context("mx_" + which, wl)
    x = dg.make_x(wl)
    xd = to_dev(wl, x)
    y = _stack(ctx, xd, wl.B)
    yn = to_np(y)
    ref = orc.stack_forward(x.astype(np.float64), wl, ws)
    err = row_err(yn, ref)
    say("mxfp8 W=512 stack err", which, err)
    assert np.all(np.isfinite(yn))
    assert err <= TOL["bf16"]
    ref_bf16 = orc.stack_forward(x.astype(np.float64), wl, ws, rho=True, mx=False)
    dev = row_err(yn, ref_bf16)
    say("mxfp8 W=512 vs bf16 path", which, dev)
    assert dev > err
    # bit-stable, and rows independent of the batch they come in
    assert torch_equal(_stack(ctx, xd, wl.B), y)
    for B in (1, 77):
        assert torch_equal(_stack(ctx, xd[:B].contiguous(), B), y[:B])
    drop("mx_" + which)


def torch_equal(a, b):
    import torch
    return bool(torch.equal(a, b))


# W = 768 (T = H = 4, D = 768): 32 experts of 3 chunks, a shared expert of
# 6 (the kernels' GEMM2 steps take 6 weight fragments at once)
MX_MOE_768 = MX_MOE_SMALL.with_(name="mx_moe_768", D=768, E=32, expert_hidden=384, shared_hidden=768, alpha=8.0)


@pytest.mark.parametrize("W", [512, 768])
@pytest.mark.parametrize("sub", [0, 1])
def test_mxfp8_moe_f_alone_zero_residual(sub, W):
    """MoE sub-layer output F alone (Revert with a zero residual; the Mix
    sub-layer's residual is its input, subtracted here in fp64), on the
    routes the GPU chose after checking them against the oracle's: the
    routed and shared experts' MXFP8 SwiGLUs within the F bounds."""
    require_gpu()
    import torch
    base = MX_MOE_SMALL if W == 512 else MX_MOE_768
    wl = base.with_(name=f"mx_moe_f{W}", L=1, B=256, down_scale=1.0, seed=47)
    ctx, banks, ws = context(f"mx_moe_f{W}", wl)
    x = dg.make_x(wl)
    xd = to_dev(wl, x)
    idx_g, gate_g = route_gpu(ctx, wl, 0, sub, xd, wl.B)
    idx_o, gate_o, logits, bound = route_oracle(wl, ws, 1, sub, x.astype(np.float64))
    nb = check_routing(wl, idx_g, gate_g, idx_o, gate_o, logits, bound)
    out = torch.empty_like(xd)
    if sub == 0:
        ctx.sublayer_forward(0, 0, xd, None, None, out, wl.B, stream())
    else:
        ctx.sublayer_forward(0, 1, xd, torch.zeros_like(xd), None, out, wl.B, stream())
    torch.cuda.synchronize()
    xf = x.astype(np.float64)
    ref = oracle_sublayer(wl, ws, 1, sub, xf, None if sub == 0 else np.zeros(x.shape), route=idx_g)
    y = to_np(out)
    if sub == 0:            # F = out - H through the same map (the rows of H are exact bf16)
        y, ref = y - xf, ref - xf
    per_row = np.max(np.abs(y - ref), axis=-1) / np.max(np.abs(ref), axis=-1)
    say("mxfp8 MoE F alone", sub, "banded routes", nb, "max", per_row.max(), "median", np.median(per_row))
    # (sub 0: y carries the bf16 rounding of H + F, 2^-9 of |H|, on top)
    slack = 0.0 if sub == 1 else 2.0 ** -8 * float(np.max(np.abs(xf)) / np.min(np.max(np.abs(ref), axis=-1)))
    assert per_row.max() <= TOL_F + slack and np.median(per_row) <= TOL_F_MEDIAN + slack


@pytest.mark.parametrize("which", ["w3", "w4"])
@pytest.mark.parametrize("sub", [0, 1])
def test_mxfp8_w512_sublayer_teacher_forced_full_batch(which, sub):
    """One sub-layer of the uneven-mixing dense stack (Mix W = 512, Revert
    W = 256, hidden 1024) and of the sparse-pertoken MoE stack (W = 512,
    E = 16, k = 4) at the full batch B = 4096 with MXFP8 GEMM operands,
    sampled rows."""
    require_gpu()
    import torch
    wl = dg.WORKLOADS[3 if which == "w3" else 4].with_(name="mx_" + which, dtype="mxfp8", L=1)
    say("mxfp8 full-batch sublayer", which, sub)
    ctx, banks, ws = context("mx_" + which, wl)
    x = dg.make_x(wl)
    xd = to_dev(wl, x)
    out = torch.empty_like(xd)
    rows = sample_rows(wl.B, 24, seed=70 + sub)
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
    say("mxfp8 full-batch sublayer err", which, sub, err)
    assert err <= TOL["bf16"]
    if sub == 1:
        drop("mx_" + which)


@pytest.mark.parametrize("W", [512, 768])
@pytest.mark.parametrize("sub", [0, 1])
def test_mxfp8_skewed_routing_and_empty_buckets(sub, W):
    """MXFP8 MoE with an always-empty bucket (expert 5: negative router
    column on positive inputs) and an all-rows bucket (expert 3, column x10:
    B = 1000 rows, 16 row tiles of one expert at W = 512, 8 tiles of 128 rows
    of the wide routed kernel at W = 768, the last one ragged), down matrices
    at full scale and, in the Revert sub-layer, a zero residual: the expert
    outputs of the all-rows bucket and the shared expert are what the
    comparison sees (F bounds)."""
    require_gpu()
    import torch
    from token_moe_amd import runner
    base = MX_MOE_SMALL if W == 512 else MX_MOE_768
    wl = base.with_(name=f"mx_skew{W}", L=1, B=1000, down_scale=1.0, seed=48)
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
    assert not np.any(idx_g == 5) and np.all(idx_g[..., 0] == 3)
    out = torch.empty_like(xd)
    if sub == 0:
        ctx.sublayer_forward(0, 0, xd, None, None, out, wl.B, stream())
    else:
        ctx.sublayer_forward(0, 1, xd, torch.zeros_like(xd), None, out, wl.B, stream())
    torch.cuda.synchronize()
    xf = x.astype(np.float64)
    rows = sample_rows(wl.B, 96, seed=80 + sub)
    ref = oracle_sublayer(wl, ws, 1, sub, xf[rows], None if sub == 0 else np.zeros(xf[rows].shape),
                          route=idx_g[rows])
    y = to_np(out)[rows]
    if sub == 0:
        y, ref = y - xf[rows], ref - xf[rows]
    per_row = np.max(np.abs(y - ref), axis=-1) / np.max(np.abs(ref), axis=-1)
    say("mxfp8 skewed", sub, "max", per_row.max(), "median", np.median(per_row))
    slack = 0.0 if sub == 1 else 2.0 ** -8 * float(np.max(np.abs(xf)) / np.min(np.max(np.abs(ref), axis=-1)))
    assert per_row.max() <= TOL_F + slack and np.median(per_row) <= TOL_F_MEDIAN + slack
    ctx.close()

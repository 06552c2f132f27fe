"""Dense stack with MXFP8 GEMM operands (TMX_MXFP8) on the GPU vs the oracle's
MXFP8 reading of the FP8 serving path (TokenMixer-Large 2.5.2).

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
from gpu_common import (TOL, context, oracle_sublayer, require_gpu, row_err, sample_rows, say,
                        stream, to_dev, to_np)

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
    for bad in (dict(D=512), dict(E=16, top_k=4, expert_hidden=256, shared_hidden=512), dict(hidden_mix=2048)):
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

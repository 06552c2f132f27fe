"""Dense stack with MXFP8 GEMM operands (TMX_MXFP8) on the GPU vs the oracle's
MXFP8 reading of the FP8 serving path (TokenMixer-Large 2.5.2).

Tolerance: the kernel and the oracle quantise the same quantities to E4M3
with the same block exponents, but from fp32 values that differ in their
last bits (fp32 norm statistics and accumulation against fp64), so a value
near a rounding boundary can take the neighbouring code: a change of one
E4M3 step (2^-3 of the value at most) in one of the W or h products of a
row, against a row sum of ~sqrt(W) such products. Together with the bf16
rounding of each sub-layer output this stays well inside the bf16 bound,
which the tests use (row-normwise 2e-2)."""
import numpy as np
import pytest

import datagen as dg
import oracle as orc
from gpu_common import (TOL, context, oracle_sublayer, require_gpu, row_err, sample_rows, say,
                        stream, to_dev, to_np)

pytestmark = pytest.mark.gpu

# W = 256 in both sub-layers (P = 16), ragged batch (1000 = 15 * 64 + 40),
# 2 and 3 hidden chunks, inter-residual at block 2
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

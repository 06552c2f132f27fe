"""tmx_sublayer_forward_noalloc against tmx_sublayer_forward.

The no-alloc entry point runs the same kernels with the MoE workspace carved
from the library's static device array instead of the context's. Its
output must equal the regular entry point's bit for bit (same kernels, same
inputs, same order), and match the oracle to the bf16 bound, on consecutive
calls -- the second with a smaller batch, so the array still holds the first
call's larger contents -- for both sub-layers of a bf16 MoE context and of an
MXFP8 one (to the MXFP8 row bound 2^-4 with F visible); the
largest batch the array holds runs, one more is rejected with an error that
names the limit; dense sub-layers (no workspace) run as before."""
import numpy as np
import pytest

import datagen as dg
from gpu_common import TOL, oracle_sublayer, require_gpu, route_gpu, row_err, say, stream, to_dev, to_np

pytestmark = pytest.mark.gpu

MOE = dg.Workload("noalloc_moe", B=600, T=4, H=4, D=128, L=1, E=16, top_k=4, expert_hidden=128,
                  shared_hidden=256, alpha=4.0, gap=0, seed=91, down_scale=1.0)
MOE_MX = MOE.with_(name="noalloc_moe_mx", D=512, expert_hidden=256, dtype="mxfp8", seed=93)
# bf16 at W 512, h_e 256: the routed experts run in the 128-row wide kernel
MOE_W512 = MOE.with_(name="noalloc_moe_w512", D=512, expert_hidden=256, seed=94)
WIDE = dg.Workload("noalloc_wide", B=8192, T=4, H=4, D=512, L=1, E=16, top_k=4, expert_hidden=128,
                   shared_hidden=128, alpha=4.0, gap=0, seed=92, down_scale=1.0)


def _both(ctx, wl, sub, xd, rd, B):
    import torch
    ref = torch.empty_like(xd[:B])
    out = torch.full_like(xd[:B], float("nan"))
    if sub == 0:
        ctx.sublayer_forward(0, 0, xd[:B], None, None, ref, B, stream())
        ctx.sublayer_forward_noalloc(0, 0, xd[:B], None, None, out, B, stream())
    else:
        ctx.sublayer_forward(0, 1, xd[:B], rd[:B], None, ref, B, stream())
        ctx.sublayer_forward_noalloc(0, 1, xd[:B], rd[:B], None, out, B, stream())
    torch.cuda.synchronize()
    return ref, out


@pytest.mark.parametrize("dtype", ["bf16", "bf16_w512", "mxfp8"])
def test_noalloc_matches_sublayer_forward_moe(dtype):
    require_gpu()
    import torch
    from token_moe_amd import runner
    wl = {"bf16": MOE, "bf16_w512": MOE_W512, "mxfp8": MOE_MX}[dtype]
    banks = dg.weight_banks(wl)
    ctx = runner.make_context(wl, banks)
    ws = dg.WeightSource(wl, banks)
    x = dg.make_x(wl)
    r = dg.make_x(wl, seed=wl.seed + 1)
    xd, rd = to_dev(wl, x).contiguous(), to_dev(wl, r).contiguous()
    for B in (600, 137):
        for sub in (0, 1):
            say("no-alloc MoE sub-layer", sub, "B", B)
            ref, out = _both(ctx, wl, sub, xd, rd, B)
            assert torch.equal(out, ref)
            idx_g, _ = route_gpu(ctx, wl, 0, sub, xd[:B].contiguous(), B)
            want = oracle_sublayer(wl, ws, 1, sub, x[:B].astype(np.float64),
                                   None if sub == 0 else r[:B].astype(np.float64), route=idx_g)
            err = row_err(to_np(out), want)
            say("no-alloc MoE err", dtype, sub, B, err)
            assert err <= (2.0 ** -4 if dtype == "mxfp8" else TOL["bf16"])
    ctx.close()


def test_noalloc_batch_limit_and_largest_batch():
    require_gpu()
    import torch
    from token_moe_amd import runner, tmx
    wl = WIDE
    banks = dg.weight_banks(wl)
    ctx = runner.make_context(wl, banks)
    xd = to_dev(wl, dg.make_x(wl)).contiguous()
    rd = to_dev(wl, dg.make_x(wl, seed=wl.seed + 1)).contiguous()
    out = torch.empty_like(xd)
    with pytest.raises(tmx.TmxError) as e:
        ctx.sublayer_forward_noalloc(0, 1, xd, rd, None, out, wl.B, stream())
    assert e.value.status == tmx.TMX_ERR_INVALID_ARG
    msg = e.value.message
    bmax = int(msg.split("B <= ")[1].split()[0].rstrip(")"))
    say("no-alloc limit message:", msg)
    assert 0 < bmax < wl.B
    with pytest.raises(tmx.TmxError):
        ctx.sublayer_forward_noalloc(0, 0, xd, None, None, out, bmax + 1, stream())
    for sub in (0, 1):
        ref, got = _both(ctx, wl, sub, xd, rd, bmax)
        assert torch.equal(got, ref)
    ctx.close()


def test_noalloc_dense_context_runs_like_sublayer_forward():
    require_gpu()
    import torch
    from token_moe_amd import runner
    wl = dg.Workload("noalloc_dense", B=300, T=4, H=2, D=128, L=1, hidden_mix=128, hidden_rev=256, gap=0,
                     seed=93, down_scale=1.0)
    ctx = runner.make_context(wl, dg.weight_banks(wl))
    xd = to_dev(wl, dg.make_x(wl)).contiguous()
    rd = to_dev(wl, dg.make_x(wl, seed=wl.seed + 1)).contiguous()
    for sub in (0, 1):
        ref, out = _both(ctx, wl, sub, xd, rd, wl.B)
        assert torch.equal(out, ref)
    ctx.close()

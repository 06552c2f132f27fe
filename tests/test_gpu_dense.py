"""Dense per-token SwiGLU block stack on the GPU vs the fp64 oracle."""
import numpy as np
import pytest

import datagen as dg
import oracle as orc
from gpu_common import (TOL, context, oracle_sublayer, require_gpu, row_err, sample_rows, say,
                        stream, to_dev, to_np)

pytestmark = pytest.mark.gpu

# small bf16 dense stack: ragged batch (300 = 2*128 + 44), H != T, W_mix 256, W_rev 128
SMALL_BF16 = dg.Workload("small_dense_bf16", B=300, T=4, H=2, D=128, L=4, hidden_mix=128,
                         hidden_rev=256, gap=2, seed=21)


def _stack(wl, ctx, x_dev, B):
    import torch
    y = torch.empty_like(x_dev)
    ctx.block_stack_forward(x_dev, y, B, stream())
    torch.cuda.synchronize()
    return y


def test_tiny_fp32_stack_all_rows():
    """Tiny dense fp32 block (B=128, T=H=4, D=32, L=1): every row, 1e-5."""
    require_gpu()
    wl = dg.WORKLOADS[1]
    say("tiny fp32 stack", wl)
    ctx, banks, ws = context("w1", wl)
    x = dg.make_x(wl)
    y = to_np(_stack(wl, ctx, to_dev(wl, x), wl.B))
    ref = orc.stack_forward(x.astype(np.float64), wl, ws)
    err = row_err(y, ref)
    say("tiny fp32 err", err)
    assert err <= TOL["f32"]


def test_small_bf16_stack_all_rows_ragged():
    require_gpu()
    wl = SMALL_BF16
    say("small bf16 dense stack", wl)
    ctx, banks, ws = context("small_dense", wl)
    x = dg.make_x(wl)
    y = to_np(_stack(wl, ctx, to_dev(wl, x), wl.B))
    ref = orc.stack_forward(x.astype(np.float64), wl, ws)
    err = row_err(y, ref)
    say("small bf16 err", err)
    assert err <= TOL["bf16"]
    # B = 1 and a ragged B give the same rows bit for bit (samples independent)
    import torch
    xd = to_dev(wl, x)
    y_full = _stack(wl, ctx, xd, wl.B)
    for B in (1, 129):
        yb = _stack(wl, ctx, xd[:B].contiguous(), B)
        assert torch.equal(yb, y_full[:B])


# odd H: the Mix sub-layer cannot pair adjacent positions in one tile; W = 768
ODD_H = dg.Workload("odd_h_dense_bf16", B=100, T=3, H=3, D=768, L=2, hidden_mix=128,
                    hidden_rev=256, gap=2, seed=23)


def test_odd_positions_stack_all_rows():
    require_gpu()
    wl = ODD_H
    say("odd-H dense stack", wl)
    ctx, banks, ws = context("odd_h", wl)
    x = dg.make_x(wl)
    y = to_np(_stack(wl, ctx, to_dev(wl, x), wl.B))
    ref = orc.stack_forward(x.astype(np.float64), wl, ws)
    err = row_err(y, ref)
    say("odd-H err", err)
    assert err <= TOL["bf16"]


# W = 256 in both sub-layers with P = 16: two 64-row workgroups per CU, tile
# ranges split per XCD, Mix positions 2m / 2m+1 alternating in the tile order;
# ragged batch (1000 = 15 * 64 + 40), 3 hidden chunks in the Revert sub-layer,
# inter-residual at block 2
W256_RAGGED = dg.Workload("w256_ragged_dense_bf16", B=1000, T=16, H=16, D=256, L=3, hidden_mix=256,
                          hidden_rev=384, gap=2, seed=33)


def test_w256_interleaved_ragged_all_rows():
    require_gpu()
    wl = W256_RAGGED
    say("W=256 ragged dense stack", wl)
    ctx, banks, ws = context("w256_ragged", wl)
    x = dg.make_x(wl)
    y = to_np(_stack(wl, ctx, to_dev(wl, x), wl.B))
    ref = orc.stack_forward(x.astype(np.float64), wl, ws)
    err = row_err(y, ref)
    say("W=256 ragged err", err)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("wid", [2, 3])
@pytest.mark.parametrize("sub", [0, 1])
def test_dense_sublayer_teacher_forced_full_batch(wid, sub):
    """One sub-layer at the full batch (the launch shape the bench times),
    oracle on sampled rows, the GPU's own input fed to both."""
    require_gpu()
    import torch
    wl = dg.WORKLOADS[wid]
    say("dense sublayer", wid, sub)
    ctx, banks, ws = context(f"w{wid}", wl)
    x = dg.make_x(wl)
    xd = to_dev(wl, x)
    out = torch.empty_like(xd)
    rows = sample_rows(wl.B, 48, seed=wid)
    if sub == 0:
        ctx.sublayer_forward(0, 0, xd, None, None, out, wl.B, stream())
        torch.cuda.synchronize()
        ref = oracle_sublayer(wl, ws, 1, 0, x[rows].astype(np.float64))
    else:
        xr = to_dev(wl, dg.make_x(wl, seed=wl.seed + 100))      # a stand-in X_rev
        ctx.sublayer_forward(0, 1, xr, xd, None, out, wl.B, stream())
        torch.cuda.synchronize()
        ref = oracle_sublayer(wl, ws, 1, 1, to_np(xr)[rows], x[rows].astype(np.float64))
    err = row_err(to_np(out)[rows], ref)
    say("dense sublayer err", wid, sub, err)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("wid", [2, 3])
def test_dense_stack_full_batch_sampled(wid):
    require_gpu()
    wl = dg.WORKLOADS[wid]
    say("dense stack", wid)
    ctx, banks, ws = context(f"w{wid}", wl)
    x = dg.make_x(wl)
    y = to_np(_stack(wl, ctx, to_dev(wl, x), wl.B))
    rows = sample_rows(wl.B, 24, seed=wid)
    ref = orc.stack_forward(x[rows].astype(np.float64), wl, ws)
    err = row_err(y[rows], ref)
    say("dense stack err", wid, err)
    assert err <= TOL["bf16"]
    assert np.all(np.isfinite(y))


def test_dense_determinism_and_chained_sublayers():
    """Two runs are bit-identical, and the chain of sub-layer calls equals the
    stack bit for bit (same kernels, same order)."""
    require_gpu()
    import torch
    wl = dg.WORKLOADS[2]
    ctx, banks, ws = context("w2", wl)
    x = to_dev(wl, dg.make_x(wl))
    y1 = _stack(wl, ctx, x, wl.B)
    y2 = _stack(wl, ctx, x, wl.B)
    assert torch.equal(y1, y2)
    cur, save = x, x
    xr = torch.empty_like(x)
    for l in range(1, wl.L + 1):
        ctx.sublayer_forward(l - 1, 0, cur, None, None, xr, wl.B, stream())
        inter = l % wl.gap == 0 and l < wl.L
        nxt = torch.empty_like(x)
        ctx.sublayer_forward(l - 1, 1, xr, cur, save if inter else None, nxt, wl.B, stream())
        if l % wl.gap == 0:
            save = nxt
        cur = nxt
    torch.cuda.synchronize()
    assert torch.equal(cur, y1)


def test_zero_down_weights_give_exact_identity():
    """With every down bank zero each block is the identity and the stack
    returns 2X (one inter-residual at l = 2 of 4), bit-exactly."""
    require_gpu()
    import torch
    from token_moe_amd import runner
    wl = SMALL_BF16
    banks = dg.weight_banks(wl)
    for key in banks:
        if key[2] == dg.K_DOWN:
            banks[key] = np.zeros_like(banks[key])
    ctx = runner.make_context(wl, banks)
    x = dg.make_x(wl)
    y = to_np(_stack(wl, ctx, to_dev(wl, x), wl.B))
    np.testing.assert_array_equal(y, 2.0 * x)
    ctx.close()


def test_state_error_before_weights():
    require_gpu()
    import torch
    from token_moe_amd import runner, tmx
    wl = SMALL_BF16
    ctx = tmx.Context(runner.config_from_workload(wl))
    x = torch.zeros((wl.B, wl.T, wl.D), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    with pytest.raises(tmx.TmxError) as e:
        ctx.block_stack_forward(x, y, wl.B, stream())
    assert e.value.status == tmx.TMX_ERR_STATE
    with pytest.raises(tmx.TmxError) as e:
        ctx.block_stack_forward(x, y, wl.B + 1, stream())
    assert e.value.status == tmx.TMX_ERR_INVALID_ARG
    with pytest.raises(tmx.TmxError) as e:
        ctx.block_stack_forward(x, x, wl.B, stream())
    assert e.value.status == tmx.TMX_ERR_INVALID_ARG
    with pytest.raises(tmx.TmxError) as e:   # wrong nbytes
        t = torch.zeros(10, dtype=torch.bfloat16)
        ctx.load_weights(0, 0, dg.K_UP, t.data_ptr(), 20)
    assert e.value.status == tmx.TMX_ERR_INVALID_ARG
    with pytest.raises(tmx.TmxError) as e:   # MoE kind on a dense context
        ctx.load_weights(0, 0, dg.K_ROUTER, t.data_ptr(), 20)
    assert e.value.status == tmx.TMX_ERR_INVALID_ARG
    ctx.close()


def test_create_beyond_device_memory_reports_oom_and_device_stays_usable():
    """A context whose activation buffers exceed the GPU's memory (B_max x T x
    D = 2^39 bf16 elements, 1 TiB per buffer; within the shape limits) fails
    with TMX_ERR_OOM and a message naming the allocation, releasing what it
    had allocated; a context created next runs a forward as before."""
    require_gpu()
    import torch
    from token_moe_amd import runner, tmx
    cfg = tmx.make_config(B_max=1 << 29, T=4, H=4, D=256, L=1, hidden_mix=256, hidden_rev=256,
                          dtype=tmx.TMX_BF16)
    free = []
    for _ in range(3):
        with pytest.raises(tmx.TmxError) as e:
            tmx.Context(cfg)
        assert e.value.status == tmx.TMX_ERR_OOM and "hipMalloc" in e.value.message
        free.append(torch.cuda.mem_get_info()[0])
    say("OOM message:", e.value.message, "free after each attempt", free)
    # (the first attempt also loads the library's device code and its static
    # arrays); later attempts leave nothing allocated
    assert abs(free[2] - free[1]) <= (16 << 20)
    wl = SMALL_BF16.with_(name="after_oom", L=1)
    banks = dg.weight_banks(wl)
    ctx = runner.make_context(wl, banks)
    x = dg.make_x(wl)
    y = to_np(_stack(wl, ctx, to_dev(wl, x), wl.B))
    ref = orc.stack_forward(x.astype(np.float64), wl, dg.WeightSource(wl, banks))
    assert row_err(y, ref) <= TOL["bf16"]
    ctx.close()

"""RankMixer block stack on the GPU vs the fp64 oracle (bf16, H = T, post-LN,
per-token GELU FFN with biases, or per-token ReLU-routed experts).
Tolerance: the bf16 bound, row-normwise 2e-2; post-LN outputs have unit
scale in every row, so no residual hides the FFN's contribution."""
import numpy as np
import pytest

import datagen as dg
import oracle as orc
from gpu_common import TOL, context, drop, require_gpu, row_err, sample_rows, say, stream, to_dev, to_np

pytestmark = pytest.mark.gpu

# ragged batch (300 = 4 * 64 + 44), 8 tokens of width 256 (dh 32), 2 hidden
# chunks, drawn LayerNorm gains and biases
SMALL_D256 = dg.Workload("rmx_small_d256", B=300, T=8, H=8, D=256, L=2, hidden_rev=256, gap=0, eps=1e-5,
                         seed=71, down_scale=1.0, block=dg.BLOCK_RANKMIXER, random_norm=True)
# width 512, 3 hidden chunks of 256, ragged batch (130 = 2 * 64 + 2)
SMALL_D512 = dg.Workload("rmx_small_d512", B=130, T=16, H=16, D=512, L=2, hidden_rev=768, gap=0, eps=1e-5,
                         seed=72, down_scale=1.0, block=dg.BLOCK_RANKMIXER, random_norm=True)


# ReLU-routed experts: 16 experts of hidden 128 per token (ragged batch), and
# 32 experts of hidden 128 with 16 tokens
SMALL_MOE16 = dg.Workload("rmx_small_moe16", B=300, T=8, H=8, D=256, L=2, E=16, expert_hidden=128, gap=0,
                          eps=1e-5, seed=73, down_scale=1.0, block=dg.BLOCK_RANKMIXER, random_norm=True)
SMALL_MOE32 = dg.Workload("rmx_small_moe32", B=130, T=16, H=16, D=256, L=2, E=32, expert_hidden=128, gap=0,
                          eps=1e-5, seed=74, down_scale=1.0, block=dg.BLOCK_RANKMIXER, random_norm=True)
# one token (T = H = 1): token mixing is the identity and S = LN_1(2 X); a
# grid of two tiles (not a multiple of 8: tiles in launch order)
SMALL_T1 = dg.Workload("rmx_small_t1", B=100, T=1, H=1, D=256, L=2, hidden_rev=256, gap=0, eps=1e-5,
                       seed=76, down_scale=1.0, block=dg.BLOCK_RANKMIXER, random_norm=True)
SMALL_T1_MOE = dg.Workload("rmx_small_t1_moe", B=100, T=1, H=1, D=256, L=2, E=16, expert_hidden=128, gap=0,
                           eps=1e-5, seed=77, down_scale=1.0, block=dg.BLOCK_RANKMIXER, random_norm=True)
SMALL = [SMALL_D256, SMALL_D512, SMALL_MOE16, SMALL_MOE32, SMALL_T1, SMALL_T1_MOE]
SMALL_IDS = ["d256", "d512", "moe16", "moe32", "t1", "t1_moe"]


def _stack(ctx, x_dev, B):
    import torch
    y = torch.empty_like(x_dev)
    ctx.block_stack_forward(x_dev, y, B, stream())
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("wl", SMALL, ids=SMALL_IDS)
def test_small_stack_all_rows(wl):
    require_gpu()
    say("RankMixer small stack", wl)
    ctx, banks, ws = context(wl.name, wl)
    x = dg.make_x(wl)
    y = to_np(_stack(ctx, to_dev(wl, x), wl.B))
    ref = orc.rankmixer_stack(x.astype(np.float64), wl, ws)
    err = row_err(y, ref)
    say("RankMixer small stack err", wl.name, err, "median",
        float(np.median(np.max(np.abs(y - ref), -1) / np.max(np.abs(ref), -1))))
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("wl", SMALL, ids=SMALL_IDS)
def test_chain_of_halves_is_the_stack_and_batch_independent(wl):
    """Sub-layer 0 then sub-layer 1 per block reproduces the fused stack bit
    for bit; two runs agree; B = 1 and a ragged B give the same rows."""
    require_gpu()
    import torch
    ctx, banks, ws = context(wl.name, wl)
    x = to_dev(wl, dg.make_x(wl))
    y1 = _stack(ctx, x, wl.B)
    assert torch.equal(y1, _stack(ctx, x, wl.B))
    cur = x
    for l in range(wl.L):
        s = torch.empty_like(x)
        ctx.sublayer_forward(l, 0, cur, None, None, s, wl.B, stream())
        nxt = torch.empty_like(x)
        ctx.sublayer_forward(l, 1, s, None, None, nxt, wl.B, stream())
        cur = nxt
    torch.cuda.synchronize()
    assert torch.equal(cur, y1)
    for B in (1, 65):
        assert torch.equal(_stack(ctx, x[:B].contiguous(), B), y1[:B])


@pytest.mark.parametrize("name", ["rankmixer_d256", "rankmixer_d512", "rankmixer_moe_d256"])
def test_full_batch_halves_teacher_forced(name):
    """Both halves at the full batch (the launch shape of the timed stack):
    S on every row (it is one rounding of a LayerNorm: at most one bf16 step
    apart where the two sides' statistics straddle a rounding boundary), the
    FFN half on sampled rows with the GPU's own S fed to the oracle."""
    require_gpu()
    import torch
    wl = dg.RANKMIXER_WORKLOADS[name]
    say("RankMixer halves", name)
    ctx, banks, ws = context(name, wl)
    x = dg.make_x(wl)
    xd = to_dev(wl, x)
    s = torch.empty_like(xd)
    ctx.sublayer_forward(0, 0, xd, None, None, s, wl.B, stream())
    out = torch.empty_like(xd)
    ctx.sublayer_forward(0, 1, s, None, None, out, wl.B, stream())
    torch.cuda.synchronize()
    s_np = to_np(s)
    tr = {}
    rows = sample_rows(wl.B, 32, seed=7)
    orc.rankmixer_block(x[rows].astype(np.float64), wl, 1, ws, rho=True, trace=tr)
    s_err = np.max(np.abs(s_np[rows] - tr[(1, "S")]))
    say("RankMixer S max abs diff", s_err)
    assert s_err <= 2.0 ** -6 * np.max(np.abs(tr[(1, "S")]))
    ref = orc.rankmixer_ffn_sublayer(s_np[rows], wl, 1, ws, rho=True)
    err = row_err(to_np(out)[rows], ref)
    say("RankMixer FFN half err", name, err)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("key", ["rankmixer_moe_d256", "moe32"])
def test_relu_gates_teacher_forced_all_rows(key):
    """The gates the expert kernel applies (tmx_relu_route on the GPU's own S)
    against ReLU(S Wr_t) in fp64 on every row: values within the fp32
    accumulation and 16-bit carry (1e-4 absolute + 2^-14 relative), and the
    active set exact wherever the oracle's logit is farther than 1e-4 from 0
    (a logit inside that band may fall on either side)."""
    require_gpu()
    import torch
    wl = dg.RANKMIXER_WORKLOADS[key] if key in dg.RANKMIXER_WORKLOADS else SMALL_MOE32
    ctx, banks, ws = context(wl.name, wl)
    xd = to_dev(wl, dg.make_x(wl))
    s = torch.empty_like(xd)
    ctx.sublayer_forward(0, 0, xd, None, None, s, wl.B, stream())
    gates = torch.empty((wl.B, wl.T, wl.E), dtype=torch.float32, device="cuda")
    ctx.relu_route(0, s, wl.B, gates, stream())
    torch.cuda.synchronize()
    s_np, g = to_np(s), gates.cpu().numpy().astype(np.float64)
    worst, band = 0.0, 0
    for t in range(wl.T):
        wr = ws(1, 1, dg.K_ROUTER, t)
        logits = s_np[:, t] @ wr
        ref = orc.relu_route(s_np[:, t], wr)
        worst = max(worst, float(np.max(np.abs(g[:, t] - ref) - 2.0 ** -14 * ref)))
        sure = np.abs(logits) > 1e-4
        band += int((~sure).sum())
        assert np.array_equal((g[:, t] > 0)[sure], (ref > 0)[sure])
    say("relu gates", key, "worst excess", worst, "band entries", band)
    assert worst <= 1e-4


def test_skipped_experts_and_silent_token():
    """Experts 3 and 7 never activate (zero router columns, so every tile
    skips them) and token 0's router is zero (every chunk skipped: its output
    is LN_2(S)); all rows against the oracle on the same weights."""
    require_gpu()
    wl = SMALL_MOE16.with_(name="rmx_moe16_dead", seed=75)
    banks = dg.weight_banks(wl)
    for (l, sub, kind), arr in banks.items():
        if kind == dg.K_ROUTER:
            arr[:, :, 3] = 0
            arr[:, :, 7] = 0
            arr[0] = 0
    say("RankMixer experts with skips", wl)
    ctx, _, ws = context(wl.name, wl, banks=banks)
    x = dg.make_x(wl)
    y = to_np(_stack(ctx, to_dev(wl, x), wl.B))
    ref = orc.rankmixer_stack(x.astype(np.float64), wl, ws)
    err = row_err(y, ref)
    say("RankMixer experts with skips err", err)
    drop(wl.name)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("name", ["rankmixer_d256", "rankmixer_d512", "rankmixer_moe_d256"])
def test_full_stack_sampled_rows(name):
    require_gpu()
    wl = dg.RANKMIXER_WORKLOADS[name]
    say("RankMixer full stack", name)
    ctx, banks, ws = context(name, wl)
    x = dg.make_x(wl)
    y = to_np(_stack(ctx, to_dev(wl, x), wl.B))
    rows = sample_rows(wl.B, 24, seed=8)
    ref = orc.rankmixer_stack(x[rows].astype(np.float64), wl, ws)
    err = row_err(y[rows], ref)
    say("RankMixer full stack err", name, err)
    drop(name)
    assert err <= TOL["bf16"]
    assert np.all(np.isfinite(y))


def test_state_and_kind_errors():
    require_gpu()
    import torch
    from token_moe_amd import runner, tmx
    wl = SMALL_D256
    ctx = tmx.Context(runner.config_from_workload(wl))
    x = torch.zeros((wl.B, wl.T, wl.D), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    with pytest.raises(tmx.TmxError) as e:          # W1 / W2 never loaded
        ctx.block_stack_forward(x, y, wl.B, stream())
    assert e.value.status == tmx.TMX_ERR_STATE
    t = torch.zeros(wl.T * wl.D * wl.hidden_rev, dtype=torch.bfloat16)
    for sub, kind in ((0, dg.K_UP), (1, dg.K_GATE), (1, dg.K_ROUTER)):
        with pytest.raises(tmx.TmxError) as e:
            ctx.load_weights(0, sub, kind, t.data_ptr(), t.numel() * 2)
        assert e.value.status == tmx.TMX_ERR_INVALID_ARG
    for B in (0, wl.B + 1):
        with pytest.raises(tmx.TmxError) as e:
            ctx.block_stack_forward(x, y, B, stream())
        assert e.value.status == tmx.TMX_ERR_INVALID_ARG
    with pytest.raises(tmx.TmxError) as e:          # a residual is not an input here
        ctx.sublayer_forward(0, 1, x, x, None, y, wl.B, stream())
    assert e.value.status == tmx.TMX_ERR_INVALID_ARG
    with pytest.raises(tmx.TmxError) as e:
        ctx.moe_route(0, 0, x, wl.B, torch.empty(1, dtype=torch.int32, device="cuda"),
                      torch.empty(1, device="cuda"), stream())
    assert e.value.status == tmx.TMX_ERR_UNSUPPORTED
    with pytest.raises(tmx.TmxError) as e:          # dense RankMixer: no router
        ctx.relu_route(0, x, wl.B, torch.empty(1, device="cuda"), stream())
    assert e.value.status == tmx.TMX_ERR_UNSUPPORTED
    ctx.close()

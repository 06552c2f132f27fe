"""Batches past 2^31 activation elements: the dense TokenMixer-Large block
(T = H = 16, D = 256, hidden 1024) and the RankMixer block (D = 256, kD =
1024), one block each, at B = 524388 (B*T*D = 2^31 + 147456; 524388 = 64 *
8193 + 36, so the last row tile is ragged). Row offsets past 2^31 elements
must be formed in 64 bits. X is drawn on the device from a seeded torch
generator (N(0, 1), rounded to bf16); rows on both sides of the 2^31-element
boundary, the first and the last rows are copied back and checked against
the oracle on the very same values."""
import numpy as np
import pytest

import datagen as dg
import oracle as orc
from gpu_common import TOL, require_gpu, row_err, say, stream, to_np

pytestmark = pytest.mark.gpu

B_LARGE = (1 << 31) // (16 * 256) + 100     # 524388 samples
CROSS = (1 << 31) // (16 * 256)             # first sample whose row starts at 2^31 elements


def _rows():
    rng = np.random.default_rng(5)
    rows = set(rng.choice(B_LARGE, 6, replace=False).tolist())
    rows.update({0, CROSS - 1, CROSS, CROSS + 1, B_LARGE - 1})
    return np.array(sorted(rows))


@pytest.mark.parametrize("family", ["tokenmixer_large", "rankmixer"])
def test_batch_past_2_31_elements(family):
    require_gpu()
    import torch
    from token_moe_amd import runner
    if family == "tokenmixer_large":
        wl = dg.WORKLOADS[2].with_(name="large_batch_tml", B=B_LARGE, L=1, gap=0)
        forward = orc.stack_forward
    else:
        wl = dg.RANKMIXER_WORKLOADS["rankmixer_d256"].with_(name="large_batch_rmx", B=B_LARGE, L=1)
        forward = orc.rankmixer_stack
    say("large batch", family, "B", wl.B, "elements", wl.B * wl.T * wl.D)
    banks = dg.weight_banks(wl)
    ctx = runner.make_context(wl, banks)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.seed + 1000)
    x = torch.randn((wl.B, wl.T, wl.D), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    say("large batch forward", family)
    ctx.block_stack_forward(x, y, wl.B, stream())
    torch.cuda.synchronize()
    rows = _rows()
    idx = torch.from_numpy(rows).cuda()
    xr = to_np(x.index_select(0, idx))
    yr = to_np(y.index_select(0, idx))
    ctx.close()
    del x, y
    torch.cuda.empty_cache()
    ref = forward(xr, wl, dg.WeightSource(wl, banks))
    err = row_err(yr, ref)
    say("large batch err", family, err)
    assert err <= TOL["bf16"]

"""The per-position F of each kernel shape, compared without the residual.

A sub-layer's output is residual + F(RMSNorm(x)), and with the pages' small
down initialisation (W_down x 0.01) the residual dominates it, so an error
in F hides inside the output comparison. Here the Revert sub-layer runs with
a zero residual, which leaves F alone (rounded to bf16 once), for every
kernel shape: the dense 4-wave kernels at W = 128, 512, 768 (W = 256 is
covered in test_gpu_mxfp8.py) and the routed + shared MoE kernels at W = 512
and 768 (at W = 768 both routed kernels: the 128-row one for expert hidden
384, the fused kernel's 64-row tile for other expert widths). Tolerance: the
bf16 bound, row-normwise 2e-2."""
import numpy as np
import pytest

import datagen as dg
from gpu_common import TOL, context, drop, oracle_sublayer, require_gpu, say, stream, to_dev, to_np

pytestmark = pytest.mark.gpu

CASES = {
    "dense_w128": dg.Workload("fa_dense_w128", B=200, T=4, H=2, D=128, L=1, hidden_mix=128, hidden_rev=256,
                              gap=0, seed=61),
    "dense_w512": dg.Workload("fa_dense_w512", B=200, T=8, H=8, D=512, L=1, hidden_mix=256, hidden_rev=384,
                              gap=0, seed=62),
    "dense_w768": dg.Workload("fa_dense_w768", B=130, T=4, H=4, D=768, L=1, hidden_mix=256, hidden_rev=256,
                              gap=0, seed=63),
    "moe_w512": dg.Workload("fa_moe_w512", B=200, T=8, H=8, D=512, L=1, E=16, top_k=4, expert_hidden=256,
                            shared_hidden=512, gap=0, seed=64),
    "moe_w768": dg.Workload("fa_moe_w768", B=130, T=4, H=4, D=768, L=1, E=32, top_k=4, expert_hidden=384,
                            shared_hidden=768, gap=0, seed=65),
    "moe_w768_he256": dg.Workload("fa_moe_w768_he256", B=300, T=4, H=4, D=768, L=1, E=16, top_k=4,
                                  expert_hidden=256, shared_hidden=384, gap=0, seed=66),
}


@pytest.mark.parametrize("name", list(CASES))
def test_f_alone_zero_residual(name):
    require_gpu()
    import torch
    wl = CASES[name]
    say("F alone", name)
    ctx, banks, ws = context("fa_" + name, wl)
    x = dg.make_x(wl)
    xd = to_dev(wl, x)
    out = torch.empty_like(xd)
    ctx.sublayer_forward(0, 1, xd, torch.zeros_like(xd), None, out, wl.B, stream())
    torch.cuda.synchronize()
    ref = oracle_sublayer(wl, ws, 1, 1, x.astype(np.float64), np.zeros(x.shape))
    y = to_np(out)
    per_row = np.max(np.abs(y - ref), axis=-1) / np.max(np.abs(ref), axis=-1)
    say("F alone", name, "max", per_row.max(), "median", np.median(per_row))
    drop("fa_" + name)
    assert per_row.max() <= TOL["bf16"]

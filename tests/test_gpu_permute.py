"""Mix / Revert on the GPU: bit-exact against the oracle (Eq. 9-15), in every
address form the kernels use (tmx_perm_form): per-element offsets, the fused
MLP's lane-constant 8-column units (its per-unit variant at W = 768, where
256 % (W/8) != 0), and the router's column cursor."""
import numpy as np
import pytest

import oracle as orc
from gpu_common import require_gpu, say, stream, to_np

pytestmark = pytest.mark.gpu

SHAPES = [(4, 4, 32, "f32"), (16, 16, 256, "bf16"), (16, 8, 256, "bf16"), (32, 32, 768, "bf16"),
          (4, 2, 128, "bf16"), (4, 4, 128, "bf16"), (8, 8, 512, "bf16"), (3, 6, 12, "f32")]


@pytest.mark.parametrize("form", [0, 1, 2])
@pytest.mark.parametrize("T,H,D,dtype", SHAPES)
def test_permute_bit_exact(T, H, D, dtype, form):
    require_gpu()
    import torch
    from token_moe_amd import tmx
    say("permute", T, H, D, dtype, "form", form)
    dh, W = D // H, T * (D // H)
    if form != 0 and (dh % 8 or W % 32):
        pytest.skip("8-column unit forms need D/H % 8 == 0 and T*D/H % 32 == 0")
    B = 150   # three 64-row chunks, the last one ragged
    cfg = tmx.make_config(B_max=B, T=T, H=H, D=D, L=1, hidden_mix=128, hidden_rev=128,
                          dtype=tmx.TMX_BF16 if dtype == "bf16" else tmx.TMX_F32)
    if dtype == "bf16" and dh % 8:
        pytest.skip("bf16 contexts need D/H % 8 == 0")
    try:
        ctx = tmx.Context(cfg)
    except tmx.TmxError as e:
        if e.status == tmx.TMX_ERR_UNSUPPORTED:
            pytest.skip(str(e))
        raise
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    idt = torch.int16 if dtype == "bf16" else torch.int32
    g = torch.Generator().manual_seed(T * 1000 + H)
    x = torch.randn((B, T, D), generator=g).to(tdt).cuda()
    mixed = torch.empty((B, H, W), dtype=tdt, device="cuda")
    back = torch.empty_like(x)
    ctx.debug_permute(x, mixed, B, 0, form, stream())
    ctx.debug_permute(mixed, back, B, 1, form, stream())
    # the Revert direction alone, from an independent mixed tensor
    m2 = torch.randn((B, H, W), generator=g).to(tdt).cuda()
    r2 = torch.empty_like(x)
    ctx.debug_permute(m2, r2, B, 1, form, stream())
    torch.cuda.synchronize()
    xn = to_np(x)
    np.testing.assert_array_equal(to_np(mixed), orc.mix(xn, H))
    np.testing.assert_array_equal(to_np(r2), orc.revert(to_np(m2), T))
    # bit patterns too (not just values)
    assert torch.equal(back.view(idt), x.view(idt))
    ctx.close()


def test_permute_rejects_bad_form():
    require_gpu()
    import torch
    from token_moe_amd import tmx
    ctx = tmx.Context(tmx.make_config(B_max=4, T=4, H=4, D=128, L=1, hidden_mix=128, hidden_rev=128))
    x = torch.zeros((4, 4, 128), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    with pytest.raises(tmx.TmxError) as e:
        ctx.debug_permute(x, y, 4, 0, 3, stream())
    assert e.value.status == tmx.TMX_ERR_INVALID_ARG
    ctx.close()

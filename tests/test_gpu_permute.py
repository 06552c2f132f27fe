"""Mix / Revert on the GPU: bit-exact against the oracle (Eq. 9-15)."""
import numpy as np
import pytest

import datagen as dg
import oracle as orc
from gpu_common import require_gpu, say, stream, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,H,D,dtype", [(4, 4, 32, "f32"), (16, 16, 256, "bf16"), (16, 8, 256, "bf16"),
                                         (32, 32, 768, "bf16"), (4, 2, 128, "bf16"), (3, 6, 12, "f32")])
def test_permute_bit_exact(T, H, D, dtype):
    require_gpu()
    import torch
    from token_moe_amd import tmx
    say("permute", T, H, D, dtype)
    B = 37
    cfg = tmx.make_config(B_max=B, T=T, H=H, D=D, L=1, hidden_mix=128, hidden_rev=128,
                          dtype=tmx.TMX_BF16 if dtype == "bf16" else tmx.TMX_F32)
    if dtype == "bf16" and (D // H) % 8:
        pytest.skip("bf16 contexts need D/H % 8 == 0")
    try:
        ctx = tmx.Context(cfg)
    except tmx.TmxError as e:
        if e.status == tmx.TMX_ERR_UNSUPPORTED:
            pytest.skip(str(e))
        raise
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    # distinct values: element index (exact in bf16 only up to 256, so use random bits)
    g = torch.Generator().manual_seed(T * 1000 + H)
    x = torch.randn((B, T, D), generator=g).to(tdt).cuda()
    mixed = torch.empty((B, H, T * D // H), dtype=tdt, device="cuda")
    back = torch.empty_like(x)
    ctx.debug_permute(x, mixed, B, 0, stream())
    ctx.debug_permute(mixed, back, B, 1, stream())
    torch.cuda.synchronize()
    xn = to_np(x)
    np.testing.assert_array_equal(to_np(mixed), orc.mix(xn, H))
    np.testing.assert_array_equal(to_np(back), xn)
    # bit patterns too (not just values)
    assert torch.equal(back.view(torch.int16 if dtype == "bf16" else torch.int32),
                       x.view(torch.int16 if dtype == "bf16" else torch.int32))
    ctx.close()

"""The model's front and back on the GPU (TokenMixer-Large summary section 2.2
Eq. 2-4 tokenizer, section 2.1 mean-pool head) against the oracle.

The tokens are the tokenizer's own output and the logit the head's, so both
comparisons see the MLPs in full (no residual hides them). Tokens: row-
normwise bf16 bound per (sample, token). Logits (one per sample): max |d| /
max |logit| over the batch within the bf16 bound. Whole model: the logits of
tmx_model_forward equal head(stack(tokenize(emb))) from the separate calls
bit for bit, and the oracle's model_forward within the bound."""
import numpy as np
import pytest

import datagen as dg
import oracle as orc
from gpu_common import TOL, require_gpu, row_err, sample_rows, say, stream, to_dev, to_np

pytestmark = pytest.mark.gpu

# ragged batch (150 = 2 * 64 + 22), ragged group widths (a half slab of 32
# columns, and a group wider than one slab), dense TokenMixer-Large stack
SMALL = dg.Workload("model_small", B=150, T=4, H=4, D=128, L=2, hidden_mix=128, hidden_rev=128, gap=2, seed=71,
                    down_scale=1.0, groups=(32, 96, 160), tok_hidden=256, head_hidden=128)
# MoE stack, D = 512
SMALL_MOE = dg.Workload("model_small_moe", B=100, T=4, H=4, D=512, L=1, E=16, top_k=4, expert_hidden=128,
                        shared_hidden=256, gap=0, seed=72, groups=(64, 256, 128), tok_hidden=512, head_hidden=256)


def logit_err(y, ref):
    return float(np.max(np.abs(y - ref)) / np.max(np.abs(ref)))


def _setup(wl, B_max=None):
    from token_moe_amd import runner
    banks = dg.weight_banks(wl)
    io = dg.io_banks(wl)
    ctx = runner.make_context(wl, banks, B_max=B_max, io_banks=io)
    allb = dict(banks)
    allb.update(io)
    return ctx, dg.WeightSource(wl, allb)


@pytest.mark.parametrize("wl", [SMALL, SMALL_MOE], ids=["dense", "moe"])
def test_tokenize_head_and_model_all_rows(wl):
    require_gpu()
    import torch
    say("model io", wl.name)
    ctx, ws = _setup(wl)
    emb = dg.make_emb(wl)
    ed = to_dev(wl, emb)
    X = torch.empty((wl.B, wl.T, wl.D), dtype=torch.bfloat16, device="cuda")
    ctx.tokenize(ed, X, wl.B, stream())
    torch.cuda.synchronize()
    Xref = orc.tokenize(emb.astype(np.float64), wl, ws, rho=True)
    err = row_err(to_np(X), Xref)
    say("tokenizer err", wl.name, err)
    assert err <= TOL["bf16"]
    # head on an independent [B, T, D] input
    Y = to_dev(wl, dg.make_x(wl, seed=wl.seed + 5))
    lg = torch.empty(wl.B, dtype=torch.float32, device="cuda")
    ctx.head(Y, lg, wl.B, stream())
    torch.cuda.synchronize()
    lref = orc.head(to_np(Y), wl, ws, rho=True)
    err = logit_err(lg.cpu().numpy().astype(np.float64), lref)
    say("head err", wl.name, err)
    assert err <= TOL["bf16"]
    # the whole model: separate calls and the fused entry agree bit for bit
    Ys = torch.empty_like(X)
    ctx.block_stack_forward(X, Ys, wl.B, stream())
    l_sep = torch.empty_like(lg)
    ctx.head(Ys, l_sep, wl.B, stream())
    l_model = torch.empty_like(lg)
    ctx.model_forward(ed, l_model, wl.B, stream())
    torch.cuda.synchronize()
    assert torch.equal(l_model, l_sep)
    if not wl.moe:
        # end to end against the oracle (dense: no routing to drift)
        ref = orc.model_forward(emb.astype(np.float64), wl, ws)
        err = logit_err(l_model.cpu().numpy().astype(np.float64), ref)
        say("model err", wl.name, err)
        assert err <= TOL["bf16"]
    else:
        # the head on the GPU's own stack output
        err = logit_err(l_model.cpu().numpy().astype(np.float64), orc.head(to_np(Ys), wl, ws, rho=True))
        say("model head-on-stack err", wl.name, err)
        assert err <= TOL["bf16"]
    # a smaller batch through the same context gives the same rows
    B2 = 37
    X2 = torch.empty((B2, wl.T, wl.D), dtype=torch.bfloat16, device="cuda")
    ctx.tokenize(ed[:B2].contiguous(), X2, B2, stream())
    torch.cuda.synchronize()
    assert torch.equal(X2, X[:B2])
    ctx.close()


def test_large_model_front_and_back_full_batch():
    """The 15B stack's front and back at the full batch (B 8192, T 32, D 768,
    31 groups of 128 / 256 / 384 columns, F 7936): tokens and logits on
    sampled rows; the stack itself is covered by the MoE tests."""
    require_gpu()
    import torch
    from token_moe_amd import tmx
    wl = dg.MODEL_WORKLOADS["model_moe_15b"]
    io = dg.io_banks(wl)
    ws = dg.WeightSource(wl, io)
    cfg = tmx.make_config(B_max=wl.B, T=wl.T, H=wl.H, D=wl.D, L=1, hidden_mix=128, hidden_rev=128)
    ctx = tmx.Context(cfg)
    from token_moe_amd import runner
    ctx.set_model_io(list(wl.groups), wl.tok_hidden, wl.head_hidden)
    for (_, _, kind), arr in io.items():
        t = runner.host_tensor(wl, arr).contiguous()
        ctx.load_io_weights(kind, t.data_ptr(), t.numel() * t.element_size())
    emb = dg.make_emb(wl)
    X = torch.empty((wl.B, wl.T, wl.D), dtype=torch.bfloat16, device="cuda")
    ctx.tokenize(to_dev(wl, emb), X, wl.B, stream())
    Y = to_dev(wl, dg.make_x(wl, seed=wl.seed + 5))
    lg = torch.empty(wl.B, dtype=torch.float32, device="cuda")
    ctx.head(Y, lg, wl.B, stream())
    torch.cuda.synchronize()
    rows = sample_rows(wl.B, 64, seed=7)
    err = row_err(to_np(X)[rows], orc.tokenize(emb[rows].astype(np.float64), wl, ws, rho=True))
    say("large tokenizer err", err)
    assert err <= TOL["bf16"]
    lref = orc.head(to_np(Y)[rows], wl, ws, rho=True)
    err = logit_err(lg.cpu().numpy().astype(np.float64)[rows], lref)
    say("large head err", err)
    assert err <= TOL["bf16"]
    ctx.close()


def test_model_io_errors():
    require_gpu()
    import torch
    from token_moe_amd import tmx
    cfg = tmx.make_config(B_max=8, T=4, H=4, D=128, L=1, hidden_mix=128, hidden_rev=128)
    ctx = tmx.Context(cfg)
    x = torch.zeros((8, 4, 128), dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros(8, dtype=torch.float32, device="cuda")
    with pytest.raises(tmx.TmxError) as e:
        ctx.head(x, lg, 8, stream())
    assert e.value.status == tmx.TMX_ERR_STATE
    with pytest.raises(tmx.TmxError) as e:
        ctx.set_model_io([32, 32], 128, 128)          # T - 1 = 3 groups needed
    assert e.value.status == tmx.TMX_ERR_INVALID_ARG
    with pytest.raises(tmx.TmxError) as e:
        ctx.set_model_io([32, 48, 32], 128, 128)      # width not a multiple of 32
    assert e.value.status == tmx.TMX_ERR_UNSUPPORTED
    ctx.set_model_io([32, 64, 32], 128, 128)
    with pytest.raises(tmx.TmxError) as e:
        ctx.set_model_io([32, 64, 32], 128, 128)
    assert e.value.status == tmx.TMX_ERR_STATE
    with pytest.raises(tmx.TmxError) as e:             # weights not loaded yet
        ctx.tokenize(torch.zeros((8, 128), dtype=torch.bfloat16, device="cuda"), x, 8, stream())
    assert e.value.status == tmx.TMX_ERR_STATE
    with pytest.raises(tmx.TmxError) as e:             # wrong size
        t = torch.zeros(10, dtype=torch.bfloat16)
        ctx.load_io_weights(dg.K_HEAD_DOWN, t.data_ptr(), 20)
    assert e.value.status == tmx.TMX_ERR_INVALID_ARG
    ctx.close()

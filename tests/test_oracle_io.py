"""Pins of the oracle's model front and back (TokenMixer-Large summary
section 2.2 Eq. 2-4: semantic group-wise tokenizer with a global token;
section 2.1 and the tokenmixerlarge README: mean pooling of the output
tokens, projection head, logit): a hand-worked example, torch float64
modules for the MLP form, and the structure the equations fix."""
import json
import os

import numpy as np
import pytest

import datagen as dg
import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


class _Cfg:
    def __init__(self, T, D, groups, tok_hidden, head_hidden):
        self.T, self.D, self.groups = T, D, tuple(groups)
        self.tok_hidden, self.head_hidden = tok_hidden, head_hidden


def _getter(tok_up, tok_down, head_up, head_down):
    def g(layer, sub, kind, p):
        return {orc.tmx_oracle._K_TOK_UP: lambda: np.asarray(tok_up[p], float),
                orc.tmx_oracle._K_TOK_DOWN: lambda: np.asarray(tok_down[p], float),
                orc.tmx_oracle._K_HEAD_UP: lambda: np.asarray(head_up, float),
                orc.tmx_oracle._K_HEAD_DOWN: lambda: np.asarray(head_down, float)}[kind]()
    return g


def test_hand_worked_tokenizer_and_head():
    g = json.load(open(os.path.join(GOLDEN, "tokenizer_head_hand.json")))
    cfg = _Cfg(g["T"], g["D"], g["groups"], g["tok_hidden"], g["head_hidden"])
    w = _getter(g["tok_up"], g["tok_down"], g["head_up"], g["head_down"])
    emb = np.asarray([g["emb"]], float)
    for rho in (False, True):
        X = orc.tokenize(emb, cfg, w, rho)
        np.testing.assert_array_equal(X[0], np.asarray(g["X"], float))
        assert orc.head(X, cfg, w, rho)[0] == g["logit"]


def test_mlp2_is_linear_relu_linear():
    import torch
    rng = np.random.default_rng(0)
    v = rng.standard_normal((9, 7))
    w1, w2 = rng.standard_normal((7, 5)), rng.standard_normal((5, 3))
    m = torch.nn.Sequential(torch.nn.Linear(7, 5, bias=False), torch.nn.ReLU(), torch.nn.Linear(5, 3, bias=False))
    m = m.double()
    with torch.no_grad():
        m[0].weight.copy_(torch.from_numpy(w1.T))
        m[2].weight.copy_(torch.from_numpy(w2.T))
        want = m(torch.from_numpy(v)).numpy()
    np.testing.assert_allclose(orc.mlp2(v, w1, w2), want, rtol=1e-13, atol=1e-13)


def _random_model(rng, groups=(3, 5, 2), D=4, h=6, hh=5):
    T = len(groups) + 1
    F = sum(groups)
    tok_up = [rng.standard_normal((F if t == 0 else groups[t - 1], h)) for t in range(T)]
    tok_down = [rng.standard_normal((h, D)) for _ in range(T)]
    return _Cfg(T, D, groups, h, hh), _getter(tok_up, tok_down, rng.standard_normal((D, hh)),
                                             rng.standard_normal(hh)), F


def test_each_group_token_reads_only_its_columns():
    """Eq. 2: token t depends on group t's columns only; Eq. 3: the global
    token (position 0, Eq. 4) on all of them. Perturbing one group moves its
    own token and the global token, nothing else (an offset or a group
    order mistake fails)."""
    rng = np.random.default_rng(1)
    cfg, w, F = _random_model(rng)
    emb = rng.standard_normal((6, F))
    X = orc.tokenize(emb, cfg, w)
    off = orc.group_offsets(cfg.groups)
    for t in range(1, cfg.T):
        e2 = emb.copy()
        e2[:, off[t - 1]:off[t]] += 1.0
        X2 = orc.tokenize(e2, cfg, w)
        changed = [u for u in range(cfg.T) if not np.array_equal(X2[:, u], X[:, u])]
        assert changed == [0, t]
    np.testing.assert_allclose(X[:, 0], orc.mlp2(emb, w(0, 0, 16, 0), w(0, 0, 17, 0)), rtol=1e-14)


def test_head_is_mean_pool_then_mlp():
    """Permuting the tokens leaves the logit unchanged (mean pooling); with
    W1 = I and w2 = 1 the logit is the sum of the positive pooled values."""
    rng = np.random.default_rng(2)
    cfg, w, F = _random_model(rng)
    Y = rng.standard_normal((5, cfg.T, cfg.D))
    l = orc.head(Y, cfg, w)
    np.testing.assert_allclose(orc.head(Y[:, rng.permutation(cfg.T)], cfg, w), l, rtol=1e-13)
    cfg2 = _Cfg(cfg.T, cfg.D, cfg.groups, cfg.tok_hidden, cfg.D)
    w_id = _getter(None, None, np.eye(cfg.D), np.ones(cfg.D))
    pooled = Y.mean(axis=1)
    np.testing.assert_allclose(orc.head(Y, cfg2, w_id), np.maximum(pooled, 0).sum(-1), rtol=1e-13)


def test_bf16_rounding_points():
    wl = dg.MODEL_WORKLOADS["model_dense"].with_(B=3, L=1)
    banks = dg.io_banks(wl)
    ws = dg.WeightSource(wl, banks)
    emb = dg.make_emb(wl).astype(np.float64)
    X = orc.tokenize(emb, wl, ws, rho=True)
    np.testing.assert_array_equal(X, orc.round_bf16(X))
    X64 = orc.tokenize(emb, wl, ws, rho=False)
    assert np.max(np.abs(X - X64)) / np.max(np.abs(X64)) < 2e-2
    assert np.all(np.isfinite(orc.head(X, wl, ws, rho=True)))


def test_io_flops_closed_form():
    wl = dg.MODEL_WORKLOADS["model_moe_15b"]
    F, h, hh = wl.emb_width, wl.tok_hidden, wl.head_hidden
    by_layer = 2 * F * h + 2 * sum(wl.groups) * h + 2 * wl.T * h * wl.D + 2 * wl.D * hh + 2 * hh
    assert orc.io_flops_per_sample(wl) == by_layer


def test_model_workload_banks_and_slices():
    wl = dg.MODEL_WORKLOADS["model_dense"].with_(B=2)
    b = dg.io_banks(wl)
    F = wl.emb_width
    assert b[(0, 0, dg.K_TOK_UP)].shape == (2 * F, wl.tok_hidden)
    ws = dg.WeightSource(wl, b)
    for t in range(wl.T):
        want = dg.io_slice(wl, dg.K_TOK_UP, t)
        np.testing.assert_array_equal(ws(0, 0, dg.K_TOK_UP, t), want)
        assert want.shape[0] == (F if t == 0 else wl.groups[t - 1])

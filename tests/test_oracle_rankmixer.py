"""Pins of the RankMixer part of the CPU oracle (layernorm, gelu, pffn,
relu_route / relu_moe, rankmixer_block / rankmixer_ffn_sublayer /
rankmixer_stack, the FLOP count).

Each is checked against something other than itself: a hand-worked block
(tests/golden/rankmixer_block_hand.json), torch's own LayerNorm / GELU /
Linear in float64, closed forms and invariants. Each test names the mistake
it would catch.
"""
import json
import math
import os

import numpy as np
import pytest

import datagen as dg
import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _phi(x):
    return 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))


def _num(s):
    return float(eval(str(s).replace("^", "**"), {"__builtins__": {}}, {"Phi": _phi}))


def _torch():
    torch = pytest.importorskip("torch")
    return torch


# ---------------------------------------------------------------------------
# layernorm
# ---------------------------------------------------------------------------

def test_layernorm_matches_torch_with_gain_and_bias():
    """Catches: unbiased variance, eps outside the root, gain/bias swapped."""
    torch = _torch()
    rng = np.random.default_rng(3)
    v = rng.standard_normal((7, 33)) * 3 + 2
    g = rng.standard_normal(33)
    b = rng.standard_normal(33)
    for eps in (1e-5, 0.3):
        got = orc.layernorm(v, g, b, eps)
        want = torch.nn.functional.layer_norm(torch.from_numpy(v), (33,), torch.from_numpy(g),
                                              torch.from_numpy(b), eps).numpy()
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_layernorm_invariants():
    """Rows of the plain LN have mean 0 and mean square var/(var+eps); a
    constant row maps to the bias (catches a missing centring)."""
    rng = np.random.default_rng(4)
    v = rng.standard_normal((5, 16)) * 2 + 7
    eps = 0.01
    y = orc.layernorm(v, None, None, eps)
    var = v.var(axis=-1)
    np.testing.assert_allclose(y.mean(axis=-1), 0, atol=1e-13)
    np.testing.assert_allclose((y * y).mean(axis=-1), var / (var + eps), rtol=1e-12)
    beta = np.arange(16.0)
    np.testing.assert_array_equal(orc.layernorm(np.full((2, 16), 3.5), np.ones(16), beta, eps), [beta, beta])


# ---------------------------------------------------------------------------
# gelu
# ---------------------------------------------------------------------------

def test_gelu_matches_torch_exact_form():
    """Catches the tanh approximation and a wrong erf argument scale."""
    torch = _torch()
    z = np.linspace(-9, 9, 1001)
    want = torch.nn.functional.gelu(torch.from_numpy(z), approximate="none").numpy()
    np.testing.assert_allclose(orc.gelu(z), want, rtol=1e-13, atol=1e-15)


def test_gelu_closed_forms():
    """GELU(0) = 0; GELU(1) = Phi(1) = 0.841344746068543 (standard normal
    table); GELU(z) - GELU(-z) = z since Phi(-z) = 1 - Phi(z)."""
    assert orc.gelu(np.array([0.0]))[0] == 0.0
    assert abs(orc.gelu(np.array([1.0]))[0] - 0.841344746068543) < 1e-14
    z = np.linspace(-5, 5, 41)
    np.testing.assert_allclose(orc.gelu(z) - orc.gelu(-z), z, atol=1e-14)


# ---------------------------------------------------------------------------
# pffn
# ---------------------------------------------------------------------------

def test_pffn_matches_torch_linear_modules():
    """Catches transposed W1 / W2 (non-square shapes) and a bias on the wrong
    side of the activation."""
    torch = _torch()
    rng = np.random.default_rng(5)
    D, kD = 6, 10
    s = rng.standard_normal((4, D))
    w1, b1 = rng.standard_normal((D, kD)), rng.standard_normal(kD)
    w2, b2 = rng.standard_normal((kD, D)), rng.standard_normal(D)
    l1 = torch.nn.Linear(D, kD).double()
    l2 = torch.nn.Linear(kD, D).double()
    with torch.no_grad():
        l1.weight.copy_(torch.from_numpy(w1.T))
        l1.bias.copy_(torch.from_numpy(b1))
        l2.weight.copy_(torch.from_numpy(w2.T))
        l2.bias.copy_(torch.from_numpy(b2))
        want = l2(torch.nn.GELU()(l1(torch.from_numpy(s)))).numpy()
    np.testing.assert_allclose(orc.pffn(s, w1, b1, w2, b2), want, rtol=1e-12, atol=1e-12)


def test_pffn_zero_first_matrix_closed_form():
    """W1 = 0: every row is GELU(b1) W2 + b2, whatever s is."""
    rng = np.random.default_rng(6)
    b1 = rng.standard_normal(5)
    w2, b2 = rng.standard_normal((5, 3)), rng.standard_normal(3)
    got = orc.pffn(rng.standard_normal((4, 3)), np.zeros((3, 5)), b1, w2, b2)
    g = np.array([x * _phi(x) for x in b1])
    np.testing.assert_allclose(got, np.tile(g @ w2 + b2, (4, 1)), rtol=1e-13)


# ---------------------------------------------------------------------------
# the block
# ---------------------------------------------------------------------------

def _golden_weights(g):
    tables = {
        (0, orc.tmx_oracle._K_GAIN): g["ln1_gain"], (0, orc.tmx_oracle._K_NBIAS): g["ln1_bias"],
        (1, orc.tmx_oracle._K_GAIN): g["ln2_gain"], (1, orc.tmx_oracle._K_NBIAS): g["ln2_bias"],
    }

    def weights(layer, sub, kind, p):
        if (sub, kind) in tables:
            return np.array(tables[(sub, kind)], dtype=np.float64)
        key = {dg.K_UP: "W1", dg.K_BIAS_UP: "b1", dg.K_DOWN: "W2", dg.K_BIAS_DOWN: "b2"}[kind]
        return np.array(g[key][p], dtype=np.float64)
    return weights


def test_block_hand_worked():
    """The hand-worked 2-token block: token mixing direction and residual,
    both LayerNorms with their own parameters, the FFN's second residual
    taken from S (not X)."""
    with open(os.path.join(GOLDEN, "rankmixer_block_hand.json")) as f:
        g = json.load(f)
    wl = dg.Workload("hand", B=1, T=2, H=2, D=2, L=1, hidden_rev=2, gap=0, eps=g["eps"],
                     dtype="f32", block=dg.BLOCK_RANKMIXER)
    X = np.array([g["X"]], dtype=np.float64)
    trace = {}
    Y = orc.rankmixer_block(X, wl, 1, _golden_weights(g), rho=False, trace=trace)
    S_want = np.array([[[_num(v) for v in row] for row in g["S"]]])
    Y_want = np.array([[[_num(v) for v in row] for row in g["Y"]]])
    np.testing.assert_allclose(trace[(1, "S")], S_want, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(Y, Y_want, rtol=1e-13, atol=1e-15)


def _torch_block(torch, X, wl, ws, layer):
    """The block written with torch modules in float64: token mixing as the
    reproduction guide's reshape + transpose, nn.LayerNorm, nn.Linear, nn.GELU."""
    B, T, D = X.shape
    H, dh = wl.H, D // wl.H
    x = torch.from_numpy(X)
    tm = x.reshape(B, T, H, dh).transpose(1, 2).reshape(B, H, T * dh)

    def ln(sub):
        m = torch.nn.LayerNorm(D, eps=wl.eps).double()
        with torch.no_grad():
            m.weight.copy_(torch.from_numpy(np.asarray(ws(layer, sub, dg.K_NORM_GAIN, 0), np.float64)))
            m.bias.copy_(torch.from_numpy(np.asarray(ws(layer, sub, dg.K_NORM_BIAS, 0), np.float64)))
        return m

    with torch.no_grad():
        S = ln(0)(tm + x)
        outs = []
        for t in range(T):
            l1 = torch.nn.Linear(D, wl.hidden_rev).double()
            l2 = torch.nn.Linear(wl.hidden_rev, D).double()
            l1.weight.copy_(torch.from_numpy(np.asarray(ws(layer, 1, dg.K_UP, t), np.float64).T))
            l1.bias.copy_(torch.from_numpy(np.asarray(ws(layer, 1, dg.K_BIAS_UP, t), np.float64)))
            l2.weight.copy_(torch.from_numpy(np.asarray(ws(layer, 1, dg.K_DOWN, t), np.float64).T))
            l2.bias.copy_(torch.from_numpy(np.asarray(ws(layer, 1, dg.K_BIAS_DOWN, t), np.float64)))
            outs.append(l2(torch.nn.GELU()(l1(S[:, t]))) + S[:, t])
        return ln(1)(torch.stack(outs, dim=1)).numpy()


def test_block_and_stack_match_torch_modules():
    """Two stacked blocks with drawn gains and biases (fp64, no rounding):
    per-token weights indexed by the right token, LN parameters per
    sub-layer and layer, blocks applied in order."""
    torch = _torch()
    wl = dg.Workload("rmx_tiny", B=3, T=4, H=4, D=8, L=2, hidden_rev=12, gap=0, eps=1e-5,
                     dtype="f32", seed=9, down_scale=1.0, block=dg.BLOCK_RANKMIXER, random_norm=True)
    ws = dg.WeightSource(wl)
    X = dg.make_x(wl).astype(np.float64)
    Y1 = _torch_block(torch, X, wl, ws, 1)
    np.testing.assert_allclose(orc.rankmixer_block(X, wl, 1, ws), Y1, rtol=1e-11, atol=1e-12)
    Y2 = _torch_block(torch, Y1, wl, ws, 2)
    np.testing.assert_allclose(orc.rankmixer_stack(X, wl, ws, rho=False), Y2, rtol=1e-10, atol=1e-11)


def test_token_mixing_is_an_involution_when_heads_equal_tokens():
    """With H = T mixing twice returns X, so the residual TM(X) + X is
    direction-free (chapter 7.4.1, H = T)."""
    X = np.random.default_rng(7).standard_normal((2, 4, 12))
    np.testing.assert_array_equal(orc.mix(orc.mix(X, 4), 4), X)


def test_block_rejects_heads_not_equal_tokens():
    wl = dg.Workload("bad", B=1, T=4, H=2, D=8, L=1, hidden_rev=8, gap=0, dtype="f32",
                     block=dg.BLOCK_RANKMIXER)
    with pytest.raises(ValueError):
        orc.rankmixer_block(np.zeros((1, 4, 8)), wl, 1, dg.WeightSource(wl))


def test_bf16_block_rounds_at_the_three_storage_points():
    """In bf16 mode S and the output are bf16 values, and the result moves
    from the unrounded one by about the bf16 step (a missing or extra
    rounding point shows as an error far outside that band)."""
    wl = dg.RANKMIXER_WORKLOADS["rankmixer_d256"].with_(B=4, L=1, random_norm=True)
    ws = dg.WeightSource(wl)
    X = dg.make_x(wl).astype(np.float64)
    tr = {}
    y = orc.rankmixer_stack(X, wl, ws, rho=True, trace=tr)
    np.testing.assert_array_equal(orc.round_bf16(y), y)
    np.testing.assert_array_equal(orc.round_bf16(tr[(1, "S")]), tr[(1, "S")])
    y0 = orc.rankmixer_stack(X, wl, ws, rho=False)
    err = np.max(np.abs(y - y0)) / np.max(np.abs(y0))
    assert 1e-4 < err < 2e-2


def test_ffn_sublayer_is_the_second_half_of_the_block():
    wl = dg.RANKMIXER_WORKLOADS["rankmixer_d256"].with_(B=3, L=1)
    ws = dg.WeightSource(wl)
    X = dg.make_x(wl).astype(np.float64)
    tr = {}
    y = orc.rankmixer_block(X, wl, 1, ws, rho=True, trace=tr)
    np.testing.assert_array_equal(orc.rankmixer_ffn_sublayer(tr[(1, "S")], wl, 1, ws, rho=True), y)


def _dense_rmx():
    return [wl for wl in dg.RANKMIXER_WORKLOADS.values() if not wl.moe]


def test_rankmixer_flops_closed_form():
    """Chapter 7.4.2: a block costs 2 T k D^2 multiply-adds (kD = hidden)."""
    for wl in _dense_rmx():
        k = wl.hidden_rev // wl.D
        assert orc.rankmixer_flops_per_sample(wl) == wl.L * 2 * (2 * wl.T * k * wl.D ** 2)


def test_rankmixer_param_count():
    """Chapter 7.4.2: per block 2 T k D^2 matrix weights, plus T (kD + D) biases."""
    for wl in _dense_rmx():
        k = wl.hidden_rev // wl.D
        assert dg.param_count(wl) == wl.L * (2 * wl.T * k * wl.D ** 2 + wl.T * (k * wl.D + wl.D))


# ---------------------------------------------------------------------------
# ReLU-routed experts (chapter 7.4.3, inference router)
# ---------------------------------------------------------------------------

def _moe_weights(rng, D, E, he):
    return (rng.standard_normal((D, E)), rng.standard_normal((E, D, he)) / np.sqrt(D),
            rng.standard_normal((E, he)), rng.standard_normal((E, he, D)) / np.sqrt(he),
            rng.standard_normal((E, D)))


def test_relu_moe_matches_sparse_torch_evaluation():
    """Row by row, only the experts with a positive gate, each a torch
    Linear-GELU-Linear scaled by its gate (catches softmax or top-k in
    place of ReLU, an ungated second bias, a wrong expert index)."""
    torch = _torch()
    rng = np.random.default_rng(11)
    D, E, he, n = 6, 5, 7, 9
    wr, w1, b1, w2, b2 = _moe_weights(rng, D, E, he)
    s = rng.standard_normal((n, D))
    v, G = orc.relu_moe(s, wr, w1, b1, w2, b2)
    want = np.zeros((n, D))
    with torch.no_grad():
        for i in range(n):
            logits = torch.from_numpy(s[i] @ wr)
            for j in range(E):
                g = float(torch.relu(logits[j]))
                if g == 0.0:
                    continue
                l1 = torch.nn.Linear(D, he).double()
                l2 = torch.nn.Linear(he, D).double()
                l1.weight.copy_(torch.from_numpy(w1[j].T)); l1.bias.copy_(torch.from_numpy(b1[j]))
                l2.weight.copy_(torch.from_numpy(w2[j].T)); l2.bias.copy_(torch.from_numpy(b2[j]))
                want[i] += g * l2(torch.nn.GELU()(l1(torch.from_numpy(s[i])))).numpy()
    np.testing.assert_allclose(v, want, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(G, np.maximum(s @ wr, 0.0))


def test_relu_moe_active_counts_vary_and_zero_router_is_silent():
    """Rows activate different numbers of experts (no fixed k); a zero
    router activates none, so the FFN contributes exactly nothing."""
    rng = np.random.default_rng(12)
    D, E, he = 8, 16, 4
    wr, w1, b1, w2, b2 = _moe_weights(rng, D, E, he)
    s = rng.standard_normal((200, D))
    _, G = orc.relu_moe(s, wr, w1, b1, w2, b2)
    counts = (G > 0).sum(axis=1)
    assert counts.min() < counts.max() and 0 < counts.mean() < E
    v0, G0 = orc.relu_moe(s, np.zeros_like(wr), w1, b1, w2, b2)
    assert not G0.any() and not v0.any()


def test_relu_moe_is_positively_homogeneous_in_the_router():
    """v(c Wr) = c v(Wr) for c > 0: the gates scale, the active set does not
    change (a normalised router -- softmax -- fails this)."""
    rng = np.random.default_rng(13)
    wr, w1, b1, w2, b2 = _moe_weights(rng, 6, 5, 3)
    s = rng.standard_normal((10, 6))
    v, _ = orc.relu_moe(s, wr, w1, b1, w2, b2)
    v3, _ = orc.relu_moe(s, 3.0 * wr, w1, b1, w2, b2)
    np.testing.assert_allclose(v3, 3.0 * v, rtol=1e-12, atol=1e-13)


def test_moe_block_with_zero_router_is_two_layernorms():
    """With every router zero the block is X' = LN_2(S), S = LN_1(TM(X) + X)."""
    wl = dg.RANKMIXER_WORKLOADS["rankmixer_moe_d256"].with_(B=3, L=1, random_norm=True)
    ws = dg.WeightSource(wl)

    def weights(layer, sub, kind, p):
        w = ws(layer, sub, kind, p)
        return np.zeros_like(w) if kind == dg.K_ROUTER else w
    X = dg.make_x(wl).astype(np.float64)
    tr = {}
    y = orc.rankmixer_block(X, wl, 1, weights, rho=False, trace=tr)
    want = orc.layernorm(tr[(1, "S")], ws(1, 1, dg.K_NORM_GAIN, 0), ws(1, 1, dg.K_NORM_BIAS, 0), wl.eps)
    np.testing.assert_allclose(y, want, rtol=1e-13, atol=1e-13)


def test_moe_workload_closed_forms():
    """Parameters per block and token: router D E, experts E (2 D h_e + h_e + D);
    FLOPs: every expert and the router on every row."""
    wl = dg.RANKMIXER_WORKLOADS["rankmixer_moe_d256"]
    D, E, he = wl.D, wl.E, wl.expert_hidden
    assert dg.param_count(wl) == wl.L * wl.T * (D * E + E * (2 * D * he + he + D))
    assert orc.rankmixer_flops_per_sample(wl) == wl.L * wl.T * 2 * (2 * D * E * he + D * E)

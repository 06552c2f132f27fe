"""Pins of the CPU oracle against the pages and plain mathematics.

Every oracle function is checked here against something other than itself:
hand-worked fixtures (tests/golden), closed forms, textbook routines (numpy
reshape/swapaxes, torch's bf16 conversion), brute-force enumeration, and
invariants the pages state. Each test names the mistake it would catch.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import datagen as dg
import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _num(s):
    """Parse the small expression language of the golden files."""
    return float(eval(s.replace("^", "**"), {"__builtins__": {}},
                      {"ln3": math.log(3.0), "inf": math.inf}))


# ---------------------------------------------------------------------------
# rho (bf16 rounding)
# ---------------------------------------------------------------------------

def test_round_bf16_hand_cases():
    g = _load("bf16_rounding.json")
    for src, want in g["cases"]:
        got = float(orc.round_bf16(_num(src)))
        assert got == _num(want), (src, got, want)


def test_round_bf16_matches_torch_on_fp32_inputs():
    # Reduces to a library routine: for fp32 inputs, rounding to bf16 is
    # torch's fp32 -> bf16 conversion (round to nearest even).
    import torch
    rng = np.random.default_rng(7)
    a = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 200000).astype(np.float32),
        # exact ties: bf16 value + half a spacing
        (np.float32(1.0) + np.arange(1, 2000, dtype=np.float32) * np.float32(2.0 ** -8)),
    ]).astype(np.float32)
    a = a[np.isfinite(a)]
    want = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    got = orc.round_bf16(a.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_round_bf16_is_idempotent_and_monotone():
    rng = np.random.default_rng(3)
    x = np.sort(rng.standard_normal(10000) * 100)
    y = orc.round_bf16(x)
    np.testing.assert_array_equal(orc.round_bf16(y), y)
    assert np.all(np.diff(y) >= 0)
    assert np.max(np.abs(y - x) / np.abs(x)) <= 2.0 ** -8 * (1 + 1e-12)


# ---------------------------------------------------------------------------
# Mix / Revert  (Eq. 9-15)
# ---------------------------------------------------------------------------

def test_mix_revert_hand_cases():
    g = _load("mix_revert_maps.json")
    for c in g["cases"]:
        X = np.array(c["X"], dtype=np.float64)[None]
        want = np.array(c["mixed"], dtype=np.float64)[None]
        got = orc.mix(X, c["H"])
        np.testing.assert_array_equal(got, want)
        np.testing.assert_array_equal(orc.revert(want, c["T"]), X)


@pytest.mark.parametrize("T,H,D", [(4, 4, 32), (16, 16, 256), (16, 8, 256), (16, 16, 512),
                                   (32, 32, 768), (3, 6, 12), (5, 1, 10), (1, 1, 8)])
def test_mix_is_textbook_reshape_swap(T, H, D):
    # Reduces to a textbook routine: reshape (T, H, dh) -> swap axes -> reshape.
    rng = np.random.default_rng(T * 100 + H)
    X = rng.standard_normal((3, T, D))
    dh = D // H
    ref = X.reshape(3, T, H, dh).swapaxes(1, 2).reshape(3, H, T * dh)
    Hm = orc.mix(X, H)
    np.testing.assert_array_equal(Hm, ref)
    # bijection: Revert(Mix(X)) == X and Mix(Revert(Hm)) == Hm bit-exactly
    np.testing.assert_array_equal(orc.revert(Hm, T), X)
    np.testing.assert_array_equal(orc.mix(orc.revert(Hm, T), H), Hm)


def test_mix_rejects_indivisible_width():
    with pytest.raises(ValueError):
        orc.mix(np.zeros((1, 4, 10)), 4)


# ---------------------------------------------------------------------------
# RMSNorm, Swish, SwiGLU, MoE hand examples
# ---------------------------------------------------------------------------

def test_rmsnorm_closed_forms():
    v = np.array([[3.0, 4.0]])
    eps = 1e-6
    r = 1.0 / math.sqrt(12.5 + eps)
    np.testing.assert_allclose(orc.rmsnorm(v, None, eps), [[3 * r, 4 * r]], rtol=1e-15)
    # output rms is 1 * (1 - O(eps)): exactly sqrt(ms / (ms + eps))
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 37))
    y = orc.rmsnorm(x, None, eps)
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), np.sqrt(ms / (ms + eps)), rtol=1e-13)
    # scale invariance up to the eps term: with eps = 0 exact for c = 2^k
    np.testing.assert_allclose(orc.rmsnorm(8.0 * x, None, 0.0), orc.rmsnorm(x, None, 0.0), rtol=1e-15)
    # gain multiplies per column
    gamma = np.arange(1, 38, dtype=np.float64)
    np.testing.assert_allclose(orc.rmsnorm(x, gamma, eps), y * gamma, rtol=1e-15)


def test_silu_closed_forms():
    z = np.array([0.0, math.log(3.0), -math.log(3.0), 50.0, -50.0, 1.0])
    s = orc.silu(z)
    assert s[0] == 0.0
    assert s[1] == pytest.approx(0.75 * math.log(3.0), rel=1e-15)
    assert s[2] == pytest.approx(-0.25 * math.log(3.0), rel=1e-15)
    assert s[3] == pytest.approx(50.0, rel=1e-15)
    assert abs(s[4]) < 1e-19
    assert s[5] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    # odd part: silu(z) - silu(-z) = z
    zz = np.linspace(-20, 20, 401)
    np.testing.assert_allclose(orc.silu(zz) - orc.silu(-zz), zz, atol=1e-13)


def test_softmax_closed_form():
    p = orc.softmax(np.array([[math.log(3.0), 0.0], [1000.0, 1000.0]]))
    np.testing.assert_allclose(p, [[0.75, 0.25], [0.5, 0.5]], rtol=1e-15)


def test_dense_sublayer_hand_example():
    g = _load("sublayer_hand.json")
    d = g["dense"]
    cfg = dg.Workload("hand", B=1, T=1, H=1, D=2, L=1, hidden_mix=1, hidden_rev=1, eps=0.0,
                      dtype="f32", gap=0)
    W = {dg.K_NORM_GAIN: np.ones(2), dg.K_UP: np.array(d["w_up"])[None],
         dg.K_GATE: np.array(d["w_gate"])[None], dg.K_DOWN: np.array(d["w_down"])[None]}

    def weights(layer, sub, kind, p):
        return W[kind] if kind == dg.K_NORM_GAIN else W[kind][p]

    x = np.array(d["x"])[None, None]
    out = orc.sublayer_positions(x, x, cfg, 1, 0, weights)
    np.testing.assert_allclose(out[0, 0], [_num(e) for e in d["expected"]], rtol=1e-15)


def test_moe_hand_example():
    g = _load("sublayer_hand.json")
    d, m = g["dense"], g["moe"]
    z = np.zeros((2, 1))
    exp_up = np.stack([np.array(d["w_up"]), z])
    exp_gate = np.stack([np.array(d["w_gate"]), z])
    exp_down = np.stack([np.array(d["w_down"]), np.zeros((1, 2))])
    sh_down = np.array([[0.0, 1.0]])
    x = np.array([m["x"]])
    y, idx, gate = orc.moe(x, np.array(m["w_router"]), exp_up, exp_gate, exp_down,
                           np.array(d["w_up"]), np.array(d["w_gate"]), sh_down,
                           m["top_k"], m["alpha"])
    assert idx.tolist() == [m["expected_idx"]]
    np.testing.assert_allclose(gate[0], [_num(v) for v in m["expected_gate"]], rtol=1e-15)
    np.testing.assert_allclose(x[0] + y[0], [_num(e) for e in m["expected"]], rtol=1e-15)


def test_swiglu_orientation_nonsquare():
    # Row-vector convention with W_up/W_gate [W, h], W_down [h, W]; written
    # element by element on a non-square case so a transposed operand fails.
    rng = np.random.default_rng(11)
    W, h = 3, 5
    v = rng.standard_normal((2, W))
    Wu, Wg, Wd = rng.standard_normal((W, h)), rng.standard_normal((W, h)), rng.standard_normal((h, W))
    want = np.zeros((2, W))
    for n in range(2):
        for k in range(W):
            acc = 0.0
            for j in range(h):
                gj = sum(v[n, i] * Wg[i, j] for i in range(W))
                uj = sum(v[n, i] * Wu[i, j] for i in range(W))
                acc += gj / (1.0 + math.exp(-gj)) * uj * Wd[j, k]
            want[n, k] = acc
    np.testing.assert_allclose(orc.swiglu(v, Wu, Wg, Wd), want, rtol=1e-12)


# ---------------------------------------------------------------------------
# router (Eq. 19-21): brute force, ties, exact arithmetic
# ---------------------------------------------------------------------------

def _brute_force_topk(l, k):
    """Enumerate all k-subsets; the unique one whose members all beat every
    non-member under the key (-l_e, e)."""
    E = len(l)
    key = lambda e: (-l[e], e)
    winners = [S for S in itertools.combinations(range(E), k)
               if all(key(a) < key(b) for a in S for b in range(E) if b not in S)]
    assert len(winners) == 1
    return sorted(winners[0], key=key)


@pytest.mark.parametrize("E,k", [(2, 1), (4, 2), (6, 3), (8, 4), (8, 1), (8, 8), (5, 4)])
def test_route_brute_force(E, k):
    rng = np.random.default_rng(E * 10 + k)
    n, W = 40, 6
    x = rng.standard_normal((n, W))
    Wr = rng.standard_normal((W, E))
    # plant exact ties in half the rows: integer-valued logits
    xi = rng.integers(-2, 3, (n, W)).astype(np.float64)
    Wi = rng.integers(-1, 2, (W, E)).astype(np.float64)
    for xx, ww in ((x, Wr), (xi, Wi)):
        idx, gate, logits, pi = orc.route(xx, ww, k, 1.5)
        for r in range(n):
            assert idx[r].tolist() == _brute_force_topk(logits[r].tolist(), k)
        np.testing.assert_allclose(pi.sum(1), 1.0, rtol=1e-14)
        np.testing.assert_allclose(gate, 1.5 * np.take_along_axis(pi, idx, 1), rtol=0)


def test_route_duplicate_columns_tie_to_lowest_index():
    # duplicated router columns give bit-identical logits: lowest index wins
    rng = np.random.default_rng(5)
    x = rng.standard_normal((30, 16))
    base = rng.standard_normal((16, 4))
    Wr = np.concatenate([base, base], axis=1)      # experts e and e+4 tie
    idx, _, _, _ = orc.route(x, Wr, 4, 2.0)
    for r in range(30):
        top = np.argsort(-(x[r] @ base), kind="stable")[:2]
        # the two best columns each appear twice; the lower copies come first
        assert idx[r].tolist() == [top[0], top[0] + 4, top[1], top[1] + 4]


def test_route_rejects_bad_k():
    with pytest.raises(ValueError):
        orc.route(np.zeros((1, 2)), np.zeros((2, 3)), 4, 1.0)


# ---------------------------------------------------------------------------
# MoE invariants
# ---------------------------------------------------------------------------

def _rand_moe(rng, W=6, E=5, he=3, hs=4):
    return dict(w_router=rng.standard_normal((W, E)), exp_up=rng.standard_normal((E, W, he)),
                exp_gate=rng.standard_normal((E, W, he)), exp_down=rng.standard_normal((E, he, W)),
                sh_up=rng.standard_normal((W, hs)), sh_gate=rng.standard_normal((W, hs)),
                sh_down=rng.standard_normal((hs, W)))


def test_moe_full_topk_is_soft_mixture():
    # top_k = E, alpha = 1: sum_e pi_e SwiGLU_e + shared (dense gated sum)
    rng = np.random.default_rng(1)
    w = _rand_moe(rng)
    x = rng.standard_normal((20, 6))
    y, _, _ = orc.moe(x, **w, top_k=5, alpha=1.0)
    logits = x @ w["w_router"]
    pi = np.exp(logits) / np.exp(logits).sum(1, keepdims=True)
    want = orc.swiglu(x, w["sh_up"], w["sh_gate"], w["sh_down"])
    for e in range(5):
        want = want + pi[:, e:e + 1] * orc.swiglu(x, w["exp_up"][e], w["exp_gate"][e], w["exp_down"][e])
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)


def test_moe_sparse_equals_dense_compute_then_mask():
    # TML-README deviation: evaluating every expert then masking the unchosen
    # ones gives the same output as sparse evaluation.
    rng = np.random.default_rng(2)
    w = _rand_moe(rng)
    x = rng.standard_normal((25, 6))
    y, idx, gate = orc.moe(x, **w, top_k=2, alpha=2.5)
    logits = x @ w["w_router"]
    pi = np.exp(logits - logits.max(1, keepdims=True))
    pi /= pi.sum(1, keepdims=True)
    ranks = np.argsort(np.argsort(-logits, axis=1, kind="stable"), axis=1, kind="stable")
    mask = ranks < 2
    all_out = np.stack([orc.swiglu(x, w["exp_up"][e], w["exp_gate"][e], w["exp_down"][e])
                        for e in range(5)], axis=1)           # [n, E, W]
    want = 2.5 * np.einsum("ne,new->nw", pi * mask, all_out) + orc.swiglu(
        x, w["sh_up"], w["sh_gate"], w["sh_down"])
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)


def test_moe_expert_relabelling_invariance():
    rng = np.random.default_rng(3)
    w = _rand_moe(rng)
    x = rng.standard_normal((25, 6))
    y, _, _ = orc.moe(x, **w, top_k=3, alpha=5 / 3)
    perm = rng.permutation(5)
    w2 = dict(w)
    w2["w_router"] = w["w_router"][:, perm]
    for kk in ("exp_up", "exp_gate", "exp_down"):
        w2[kk] = w[kk][perm]
    y2, _, _ = orc.moe(x, **w2, top_k=3, alpha=5 / 3)
    np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-14)


def test_moe_linear_in_alpha_without_shared():
    rng = np.random.default_rng(4)
    w = _rand_moe(rng)
    for kk in ("sh_up", "sh_gate", "sh_down"):
        w[kk] = np.zeros_like(w[kk])
    x = rng.standard_normal((25, 6))
    y1, _, _ = orc.moe(x, **w, top_k=2, alpha=1.0)
    y3, _, _ = orc.moe(x, **w, top_k=2, alpha=3.0)
    np.testing.assert_allclose(y3, 3.0 * y1, rtol=1e-13, atol=1e-15)


def test_moe_route_override():
    """The routing override: its own top-k reproduces the plain result bit for
    bit; any other set of k experts gives alpha * sum over that set of pi_e
    SwiGLU_e + shared, with pi still the softmax over all E (a mistake that
    renormalised the gates or kept the oracle's own set would fail)."""
    rng = np.random.default_rng(5)
    w = _rand_moe(rng)
    x = rng.standard_normal((12, 6))
    y, idx, gate = orc.moe(x, **w, top_k=2, alpha=2.5)
    y1, idx1, gate1 = orc.moe(x, **w, top_k=2, alpha=2.5, idx_override=idx)
    assert np.array_equal(y1, y) and np.array_equal(idx1, idx) and np.array_equal(gate1, gate)
    other = np.stack([(idx[:, 0] + 1) % 5, (idx[:, 0] + 3) % 5], axis=1)
    y2, idx2, gate2 = orc.moe(x, **w, top_k=2, alpha=2.5, idx_override=other)
    logits = x @ w["w_router"]
    pi = np.exp(logits) / np.exp(logits).sum(1, keepdims=True)
    want = orc.swiglu(x, w["sh_up"], w["sh_gate"], w["sh_down"])
    for r in range(x.shape[0]):
        for e in other[r]:
            want[r] += 2.5 * pi[r, e] * orc.swiglu(x[r:r + 1], w["exp_up"][e], w["exp_gate"][e],
                                                   w["exp_down"][e])[0]
    np.testing.assert_allclose(y2, want, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(idx2, other)
    np.testing.assert_allclose(gate2, 2.5 * np.take_along_axis(pi, other, 1), rtol=1e-13)


def test_weight_banks_kind_filter_shares_draws():
    """Two workloads that differ only in down_scale draw the same banks except
    the down matrices, which differ exactly by the factor before rounding."""
    a = dg.WORKLOADS[4].with_(L=1, B=8, T=2, H=2, D=32, E=16, expert_hidden=128, shared_hidden=128)
    b = a.with_(down_scale=1.0)
    ba = dg.weight_banks(a)
    bd = dg.weight_banks(b, kinds=dg.DOWN_KINDS)
    assert set(bd) == {k for k in ba if k[2] in dg.DOWN_KINDS}
    full_b = dg.weight_banks(b)
    for k in full_b:
        if k[2] in dg.DOWN_KINDS:
            np.testing.assert_array_equal(bd[k], full_b[k])
        else:
            np.testing.assert_array_equal(ba[k], full_b[k])


# ---------------------------------------------------------------------------
# stack wiring (Pre-Norm block, residual to block input, inter-residual)
# ---------------------------------------------------------------------------

def _zero_down(getter, subs=(0, 1)):
    downs = (dg.K_DOWN, dg.K_EXP_DOWN, dg.K_SH_DOWN)

    def g(layer, sub, kind, p):
        w = getter(layer, sub, kind, p)
        return np.zeros_like(w) if (kind in downs and sub in subs) else w
    return g


SMALL = {
    "dense": dg.Workload("small_dense", B=6, T=4, H=2, D=8, L=4, hidden_mix=12, hidden_rev=10,
                         dtype="bf16", seed=9),
    "moe": dg.Workload("small_moe", B=6, T=4, H=4, D=8, L=8, E=4, top_k=2, expert_hidden=6,
                       shared_hidden=5, alpha=2.0, dtype="bf16", seed=10),
    "tiny": dg.Workload("tiny1", B=5, T=4, H=4, D=32, L=1, hidden_mix=64, hidden_rev=64,
                        dtype="f32", seed=0),
}


@pytest.mark.parametrize("name,mult", [("dense", 2.0), ("moe", 8.0), ("tiny", 1.0)])
def test_zero_down_makes_every_block_identity(name, mult):
    # Every F = 0 => Z_l = Y_{l-1}; inter-residuals double the stream at
    # l = 2, 4, 6 (< L): Y_L = 2^{#inter} X bit-exactly (L=1: X, 4: 2X, 8: 8X)
    cfg = SMALL[name]
    X = dg.make_x(cfg).astype(np.float64)
    Y = orc.stack_forward(X, cfg, _zero_down(dg.WeightSource(cfg)))
    np.testing.assert_array_equal(Y, mult * X)


@pytest.mark.parametrize("name,mult", [("dense", 2.0), ("moe", 8.0)])
def test_revert_residual_goes_to_block_input(name, mult):
    # Mix sub-layer active, revert sub-layer F = 0: with the residual to the
    # block input X (TML Eq. 16) every block is exactly the identity. The
    # other reading (residual to X_rev) would leak the mix sub-layer's F.
    cfg = SMALL[name]
    X = dg.make_x(cfg).astype(np.float64)
    Y = orc.stack_forward(X, cfg, _zero_down(dg.WeightSource(cfg), subs=(1,)))
    np.testing.assert_array_equal(Y, mult * X)


def test_single_token_single_head_reduces_to_nested_prenorm_mlp():
    # T = H = 1: Mix and Revert are the identity, so one block is
    # X + F_rev(N(X + F_mix(N(X)))) -- written here with a plain einsum
    # formulation of SwiGLU.
    cfg = dg.Workload("t1", B=7, T=1, H=1, D=6, L=1, hidden_mix=5, hidden_rev=4, dtype="f32", seed=12)
    ws = dg.WeightSource(cfg)
    X = dg.make_x(cfg).astype(np.float64)

    def f(v, sub):
        Wu, Wg, Wd = (ws(1, sub, k, 0).astype(np.float64) for k in (dg.K_UP, dg.K_GATE, dg.K_DOWN))
        n = v / np.sqrt(np.mean(v ** 2, -1, keepdims=True) + cfg.eps)
        g = np.einsum("bi,ij->bj", n, Wg)
        u = np.einsum("bi,ij->bj", n, Wu)
        return np.einsum("bj,jk->bk", g / (1 + np.exp(-g)) * u, Wd)

    x = X[:, 0]
    h1 = x + f(x, 0)
    want = x + f(h1, 1)
    Y = orc.stack_forward(X, cfg, ws)
    np.testing.assert_allclose(Y[:, 0], want, rtol=1e-13, atol=1e-15)


def test_which_elements_change_follows_revert_map():
    # Only mixed position h* has a non-zero down bank: after the mix
    # sub-layer and Revert, only columns h*·dh..(h*+1)·dh of every token may
    # differ from the block input (TML Eq. 13-15).
    cfg = dg.Workload("wc", B=4, T=4, H=2, D=8, L=1, hidden_mix=6, hidden_rev=6, dtype="f32", seed=13)
    ws = dg.WeightSource(cfg)
    hstar, dh = 1, cfg.D // cfg.H

    def g(layer, sub, kind, p):
        w = ws(layer, sub, kind, p)
        return np.zeros_like(w) if (kind == dg.K_DOWN and p != hstar) else w

    X = dg.make_x(cfg).astype(np.float64)
    Hm = orc.mix(X, cfg.H)
    Hn = orc.sublayer_positions(Hm, Hm, cfg, 1, 0, g)
    Xr = orc.revert(Hn, cfg.T)
    changed = np.any(Xr != X, axis=(0, 1))
    assert changed[hstar * dh:(hstar + 1) * dh].all()
    assert not changed[:hstar * dh].any() and not changed[(hstar + 1) * dh:].any()


def test_inter_residual_positions():
    # With the revert F = 0 but a marker added through "extra", the
    # inter-residual must enter at l = 2, 4, 6 only (gap 2, never at l = L).
    cfg = SMALL["moe"].with_(L=6, gap=2)
    X = dg.make_x(cfg).astype(np.float64)
    Y = orc.stack_forward(X, cfg, _zero_down(dg.WeightSource(cfg)))
    np.testing.assert_array_equal(Y, 4.0 * X)            # l=2: 2X, l=4: 4X, l=6 = L: none
    cfg3 = SMALL["dense"].with_(L=6, gap=3)
    Y3 = orc.stack_forward(dg.make_x(cfg3).astype(np.float64), cfg3,
                           _zero_down(dg.WeightSource(cfg3)))
    np.testing.assert_array_equal(Y3, 2.0 * dg.make_x(cfg3))   # l=3 only
    cfg0 = SMALL["dense"].with_(gap=0)
    Y0 = orc.stack_forward(dg.make_x(cfg0).astype(np.float64), cfg0, _zero_down(dg.WeightSource(cfg0)))
    np.testing.assert_array_equal(Y0, dg.make_x(cfg0))


@pytest.mark.parametrize("name", ["dense", "moe"])
def test_samples_are_independent(name):
    cfg = SMALL[name]
    ws = dg.WeightSource(cfg)
    X = dg.make_x(cfg).astype(np.float64)
    Y = orc.stack_forward(X, cfg, ws)
    sub = [4, 1]
    np.testing.assert_array_equal(orc.stack_forward(X[sub], cfg, ws), Y[sub])


def test_bf16_mode_outputs_are_bf16_values():
    cfg = SMALL["moe"]
    Y = orc.stack_forward(dg.make_x(cfg).astype(np.float64), cfg, dg.WeightSource(cfg))
    np.testing.assert_array_equal(orc.round_bf16(Y), Y)


def test_bf16_and_fp64_modes_agree_to_bf16_precision():
    cfg = SMALL["dense"]
    ws = dg.WeightSource(cfg)
    X = dg.make_x(cfg).astype(np.float64)
    a = orc.stack_forward(X, cfg, ws, rho=True)
    b = orc.stack_forward(X, cfg, ws, rho=False)
    err = np.max(np.abs(a - b), axis=-1) / np.max(np.abs(b), axis=-1)
    assert err.max() < 2e-2 and err.max() > 0


# ---------------------------------------------------------------------------
# closed forms of the work (RMX-BOOK 7.4.2; TML 3.4 scale)
# ---------------------------------------------------------------------------

def test_param_counts():
    for i, cfg in dg.WORKLOADS.items():
        assert orc.param_count_closed_form(cfg) == dg.param_count(cfg)
    assert orc.param_count_closed_form(dg.WORKLOADS[5]) == 15_414_067_200   # the ~15B model
    assert 15e9 <= orc.param_count_closed_form(dg.WORKLOADS[5]) < 16e9
    assert orc.param_count_closed_form(dg.WORKLOADS[4]) == 1_814_036_480
    assert orc.param_count_closed_form(dg.WORKLOADS[2]) == 100_663_296
    assert orc.param_count_closed_form(dg.WORKLOADS[3]) == 100_663_296


def test_flops_equal_params_for_dense_pertoken():
    # Per-token FFN: Param = FLOPs (in multiply-adds) per sample (RMX-BOOK 7.4.2)
    for i in (1, 2, 3):
        cfg = dg.WORKLOADS[i]
        assert orc.flops_per_sample(cfg) == 2 * orc.param_count_closed_form(cfg)
    assert orc.flops_per_sample(dg.WORKLOADS[2]) == 201_326_592
    assert orc.flops_per_sample(dg.WORKLOADS[4]) == 1_212_153_856
    assert orc.flops_per_sample(dg.WORKLOADS[5]) == 5_460_983_808


# ---------------------------------------------------------------------------
# MXFP8 operands of the FP8 serving path (TML 2.5.2): E4M3 elements checked
# against torch's float8_e4m3fn (an independent implementation of the OCP
# format) and the format's published extreme values; MX block scaling
# against its defining properties
# ---------------------------------------------------------------------------

def test_e4m3_decode_matches_torch_and_format_extremes():
    import torch
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = orc.e4m3_value(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.isnan(got[[0x7F, 0xFF]]).all() and np.isnan(got).sum() == 2
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0          # largest normal
    assert got[0x08] == 2.0 ** -6 and got[0x07] == 0.875 * 2.0 ** -6   # smallest normal, largest subnormal
    assert got[0x01] == 2.0 ** -9 and got[0x38] == 1.0 and got[0x00] == 0.0


def test_e4m3_round_matches_torch_and_saturates():
    import torch
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(100000) * np.exp2(rng.integers(-14, 9, 100000))).astype(np.float32)
    x = np.clip(x, -448, 448).astype(np.float32)
    # exact midpoints between neighbouring codes (ties go to the even code)
    v = orc.e4m3_value(np.arange(0x7F))
    mid = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mid, -mid, v.astype(np.float32)])
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.e4m3_round(x)
    assert np.array_equal(got, want)
    big = np.array([448.0, 449.0, 464.0, 480.0, 1e6, 3e38], np.float32)
    assert (orc.e4m3_round(big) == 0x7E).all() and (orc.e4m3_round(-big) == 0xFE).all()


def test_mx_exponent_cases():
    # the block maximum lands in [2**8, 2**9) after scaling
    amax = np.array([1.0, 448.0, 256.0, 255.99, 511.9, 2.0 ** -20, 3e-30, 1e38, 0.0])
    assert orc.mx_exponent(amax).tolist() == [-8, 0, 0, -1, 0, -28, -107, 118, -127]
    a = np.exp2(np.random.default_rng(3).uniform(-100, 100, 1000))
    k = orc.mx_exponent(a)
    assert ((a / np.exp2(k) >= 256) & (a / np.exp2(k) < 512)).all()


def test_mx_quantize_blocks_error_bound_and_axis():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((7, 96)).astype(np.float32)
    codes, k = orc.mx_quantize(x)
    assert codes.shape == x.shape and k.shape == (7, 3)
    # blocks along the last axis are independent: scaling one block by 2**s
    # moves only its exponent
    y = x.copy()
    y[2, 32:64] *= np.float32(2.0 ** 13)
    c2, k2 = orc.mx_quantize(y)
    assert np.array_equal(c2, codes)
    d = k2 - k
    assert d[2, 1] == 13 and np.count_nonzero(d) == 1
    # values already on the block's grid come back exactly
    q = orc.mx_round(x)
    assert np.array_equal(orc.mx_round(q), q)
    # round to nearest: at most half a step of the E4M3 grid (relative 2**-4
    # for normal values, 2**-10 * 2**k below the smallest normal), except
    # values above 448 * 2**k, which saturate
    s = np.repeat(np.exp2(k.astype(np.float64)), 32, axis=1)
    r = np.abs(x.astype(np.float64)) / s
    err = np.abs(q - x) / s
    normal = (r >= 2.0 ** -6) & (r <= 448)
    assert (err[normal] <= 2.0 ** (np.floor(np.log2(r[normal])) - 4) + 1e-12).all()
    assert (err[r < 2.0 ** -6] <= 2.0 ** -10 + 1e-15).all()
    assert (np.abs(q[r > 448]) / s[r > 448] == 448).all()
    # rows of very different magnitude each keep their own scale only if the
    # blocks run along the last axis: row-normwise error at most 1/8 (a
    # block maximum in (448, 512) * 2**k saturates to 448 * 2**k); blocks
    # across rows would flush the small rows to zero
    m = (rng.standard_normal((4, 64)) * np.exp2(np.array([-30.0, -5.0, 10.0, 40.0]))[:, None]).astype(np.float32)
    rel = np.max(np.abs(orc.mx_round(m) - m), axis=1) / np.max(np.abs(m), axis=1)
    assert rel.max() <= 0.125 + 1e-9


def test_swiglu_mx_close_to_exact_with_skewed_columns():
    """The quantised SwiGLU stays within the fp8 error of the exact one even
    when weight columns and input rows differ by many binades, which only
    holds if every operand is blocked along its contraction axis."""
    rng = np.random.default_rng(13)
    W, h, n = 64, 96, 40
    v = rng.standard_normal((n, W)) * np.exp2(rng.integers(-20, 20, (n, 1)))
    wg = rng.standard_normal((W, h)) / 8 * np.exp2(rng.integers(-12, 12, (1, h)))
    wu = rng.standard_normal((W, h)) / 8 * np.exp2(rng.integers(-12, 12, (1, h)))
    wd = rng.standard_normal((h, W)) / 8 * np.exp2(rng.integers(-12, 12, (1, W)))
    # keep the hidden activations O(1)-scaled per row so silu stays in range
    v = v / np.max(np.abs(v), axis=1, keepdims=True)
    exact = orc.swiglu(v, wu, wg, wd)
    q = orc.swiglu_mx(v, wu, wg, wd)
    # compare column-normwise: the down columns carry their own scales
    err = np.max(np.abs(q - exact), axis=0) / np.max(np.abs(exact), axis=0)
    assert err.max() < 0.15 and err.max() > 1e-4


def test_mxfp8_stack_is_the_dense_stack_within_fp8_error():
    cfg = dg.Workload("mx_small", B=24, T=4, H=2, D=64, L=2, hidden_mix=64, hidden_rev=96,
                      gap=2, dtype="mxfp8", seed=17)
    ws = dg.WeightSource(cfg)
    X = dg.make_x(cfg).astype(np.float64)
    a = orc.stack_forward(X, cfg, ws)                 # MXFP8 GEMMs, bf16 outputs
    b = orc.stack_forward(X, cfg, ws, rho=True, mx=False)
    err = np.max(np.abs(a - b), axis=-1) / np.max(np.abs(b), axis=-1)
    assert 0 < err.max() < 5e-2


def _exact_mx_moe(rng, n=48, W=64, E=4, he=32, hs=64):
    """A MoE whose every GEMM operand and product is exact in MXFP8 and fp64:
    rows in {0, +-1/2, +-1} with column 0 = 1, gate weights 128 in row 0 only
    (g = 128, silu(128) = 128 in fp64), one +-1 per up column, down weights in
    {0, +-1/2, +-1}; the router is random."""
    x = rng.choice([-1.0, -0.5, 0.0, 0.5, 1.0], size=(n, W))
    x[:, 0] = 1.0

    def bank(h, lead=()):
        gate = np.zeros(lead + (W, h))
        gate[..., 0, :] = 128.0
        up = np.zeros(lead + (W, h))
        rows = rng.integers(0, W, lead + (h,))
        np.put_along_axis(up, rows[..., None, :], rng.choice([-1.0, 1.0], lead + (1, h)), axis=-2)
        down = rng.choice([-1.0, -0.5, 0.0, 0.5, 1.0], size=lead + (h, W))
        return up, gate, down

    eu, eg, ed = bank(he, (E,))
    su, sg, sd = bank(hs)
    w = dict(w_router=rng.standard_normal((W, E)), exp_up=eu, exp_gate=eg, exp_down=ed,
             sh_up=su, sh_gate=sg, sh_down=sd)
    return x, w


def test_moe_mx_exact_operands_reproduce_exact_moe():
    """With operands the MXFP8 grid holds exactly, the MXFP8 MoE equals the
    exact one bit for bit: the quantised experts are the same experts, gated
    by the same alpha * pi, plus the quantised shared expert (a wrong expert,
    gate or a dropped shared term fails)."""
    rng = np.random.default_rng(21)
    x, w = _exact_mx_moe(rng)
    y, idx, gate = orc.moe(x, **w, top_k=2, alpha=2.0)
    ym, idxm, gatem = orc.moe(x, **w, top_k=2, alpha=2.0, mx=True)
    assert np.array_equal(idxm, idx) and np.array_equal(gatem, gate)
    assert np.array_equal(ym, y)
    assert len(np.unique(idx)) == 4                    # every expert took rows


def test_moe_mx_routes_on_unquantised_rows_and_stays_within_fp8_error():
    """On general data the MXFP8 MoE keeps the exact router's choice and gates
    (the router reads xhat itself) and differs from the exact MoE by no more
    than the fp8 rounding of its operands allows."""
    rng = np.random.default_rng(22)
    W, E, he, hs, n = 64, 6, 64, 96, 60
    w = dict(w_router=rng.standard_normal((W, E)), exp_up=rng.standard_normal((E, W, he)) / 8,
             exp_gate=rng.standard_normal((E, W, he)) / 8, exp_down=rng.standard_normal((E, he, W)) / 8,
             sh_up=rng.standard_normal((W, hs)) / 8, sh_gate=rng.standard_normal((W, hs)) / 8,
             sh_down=rng.standard_normal((hs, W)) / 8)
    x = rng.standard_normal((n, W))
    y, idx, gate = orc.moe(x, **w, top_k=3, alpha=2.0)
    ym, idxm, gatem = orc.moe(x, **w, top_k=3, alpha=2.0, mx=True)
    assert np.array_equal(idxm, idx) and np.array_equal(gatem, gate)
    # E4M3 keeps 3 mantissa bits (rounding up to 2**-4 relative per operand);
    # through two chained contractions of 64 terms the row-normwise error
    # sits near 7 % with a tail to about 15 %, while a dropped expert or
    # shared term moves rows by their whole size
    err = np.max(np.abs(ym - y), axis=1) / np.max(np.abs(y), axis=1)
    assert 1e-3 < np.median(err) < 0.1 and err.max() < 0.25
    # the routed part alone: the MXFP8 SwiGLU of each chosen expert, gated
    want = orc.swiglu_mx(x, w["sh_up"], w["sh_gate"], w["sh_down"])
    for r in range(n):
        for s in range(3):
            e = idx[r, s]
            want[r] += gate[r, s] * orc.swiglu_mx(x[r:r + 1], w["exp_up"][e], w["exp_gate"][e],
                                                 w["exp_down"][e])[0]
    np.testing.assert_allclose(ym, want, rtol=1e-12, atol=1e-12)


def test_mxfp8_moe_stack_is_the_bf16_stack_within_fp8_error():
    """MXFP8 MoE stack against the bf16 one on the same inputs: the residual
    stream carries the fp8 error of the sub-layer outputs only (a row whose
    two largest logits sit within that perturbation could route differently
    in a later sub-layer; this seed has none that moves a row past 5 %)."""
    cfg = dg.Workload("mx_moe_small", B=24, T=4, H=2, D=64, L=2, E=4, top_k=2,
                      expert_hidden=64, shared_hidden=64, alpha=2.0, gap=2,
                      dtype="mxfp8", seed=23)
    ws = dg.WeightSource(cfg)
    X = dg.make_x(cfg).astype(np.float64)
    a = orc.stack_forward(X, cfg, ws)
    b = orc.stack_forward(X, cfg, ws, rho=True, mx=False)
    err = np.max(np.abs(a - b), axis=-1) / np.max(np.abs(b), axis=-1)
    assert 0 < err.max() < 5e-2


def test_sublayer_positions_subset_equals_full_evaluation():
    """Evaluating a subset of positions gives those positions' outputs of the
    full evaluation bit for bit and marks the others NaN."""
    cfg = dg.Workload("sub_pos", B=6, T=4, H=4, D=64, L=1, E=4, top_k=2, expert_hidden=64,
                      shared_hidden=64, alpha=2.0, gap=0, dtype="mxfp8", seed=24)
    ws = dg.WeightSource(cfg)
    x = dg.make_x(cfg).astype(np.float64)
    full = orc.sublayer_positions(x, x, cfg, 1, 1, ws, rho=True, mx=True)
    part = orc.sublayer_positions(x, x, cfg, 1, 1, ws, rho=True, mx=True, positions=(1, 3))
    assert np.array_equal(part[:, [1, 3]], full[:, [1, 3]])
    assert np.isnan(part[:, [0, 2]]).all()

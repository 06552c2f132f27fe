"""Plain, slow fp64 CPU oracle of the TokenMixer-Large block-stack forward.

TEST INFRASTRUCTURE ONLY. It exists to check the HIP path; it is imported by
``tests/``, by ``__graft_entry__.smoke()`` and by ``bench.py``'s cpu_baseline
leg, and by nothing else. It shares no code with the HIP library: every index
map and formula below is written out again from the pages.

Citations name the page and the equation / section / table they follow:

* [TML] "TokenMixer-Large: Scaling Up Large Ranking Models in Industrial
  Recommenders", the paper-archivist summary (sections 2.3-2.4, Eq. 9-21).
* [TML-README] the fay85/tokenmixerlarge README (block diagram in Pre-Norm
  form, flag table, documented deviations).
* [RMX-GUIDE] the samxiexs/RankMixer reproduction guide (section 5 token
  mixing constraints, section 6.1 per-token weight layout).
* [RMX-BOOK] the fun-rec mdbook chapter 7.4 on RankMixer (7.4.1, 7.4.2).

Precision contract (the pages fix none; this is the plainest reading): all
arithmetic is fp64. In bf16 mode the value is rounded to bf16 (round to
nearest, ties to even) exactly at the storage points the GPU path has:
the normalised rows x_hat, the SwiGLU hidden U, and each sub-layer output
(residual + F [+ inter-residual]) rounded once. Everything else (norm
statistics, router logits, softmax, gates, down outputs, the combine and the
residual sums) stays unrounded.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
something other than itself (closed forms, textbook routines, brute force,
hand-worked fixtures under ``tests/golden/``). No function is unpinned.
"""
from __future__ import annotations

import math
from typing import Callable, Dict, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "round_bf16", "mix", "revert", "rmsnorm", "silu", "softmax", "swiglu",
    "route", "moe", "sublayer_positions", "block_forward", "stack_forward",
    "flops_per_sample", "param_count_closed_form",
    "E4M3_MAX", "MX_BLOCK", "e4m3_value", "e4m3_round", "mx_exponent", "mx_quantize",
    "mx_dequantize", "mx_round", "swiglu_mx",
    "layernorm", "gelu", "pffn", "rankmixer_block", "rankmixer_ffn_sublayer", "rankmixer_stack",
    "rankmixer_flops_per_sample", "relu_route", "relu_moe",
    "relu", "mlp2", "group_offsets", "tokenize", "head", "model_forward", "io_flops_per_sample",
]

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


# ---------------------------------------------------------------------------
# rounding point
# ---------------------------------------------------------------------------

def round_bf16(x) -> np.ndarray:
    """rho(x): nearest bfloat16 value of fp64 x, ties to even, as fp64.

    bfloat16 keeps 8 significant bits (1 implicit + 7 stored) and the fp32
    exponent range, so a normal value m * 2**e (0.5 <= |m| < 1) is quantised
    to a multiple of 2**(e - 8); subnormals to multiples of 2**-133.
    """
    x = np.asarray(x, dtype=np.float64)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)
    q = np.maximum(e - 8, -133)
    y = np.ldexp(np.rint(np.ldexp(xf, -q)), q)       # exact scaling; rint = half-even
    y = np.where(np.abs(y) > BF16_MAX, np.copysign(np.inf, y), y)
    return np.where(finite, y, x)


def _rho(x, on: bool):
    return round_bf16(x) if on else x


# ---------------------------------------------------------------------------
# Mix / Revert   [TML] Eq. 9-11 and Eq. 13-15
# ---------------------------------------------------------------------------

def mix(X: np.ndarray, H: int) -> np.ndarray:
    """Mixing: split every token into H heads of width dh = D/H (Eq. 9); mixed
    token h concatenates head h of tokens 1..T (Eq. 10); stacking gives
    H in R^{H x T*D/H} (Eq. 11). Per sample:
    Hm[h, t*dh + j] = X[t, h*dh + j].
    D must be a multiple of H ([RMX-GUIDE] section 5)."""
    B, T, D = X.shape
    if D % H:
        raise ValueError("D must be divisible by H")
    dh = D // H
    out = np.empty((B, H, T * dh), dtype=X.dtype)
    for h in range(H):
        for t in range(T):
            out[:, h, t * dh:(t + 1) * dh] = X[:, t, h * dh:(h + 1) * dh]
    return out


def revert(Hm: np.ndarray, T: int) -> np.ndarray:
    """Reverting: split every mixed token into T pieces of width dh (Eq. 13);
    token t concatenates piece t of mixed tokens 1..H (Eq. 14-15). Per sample:
    X_rev[t, h*dh + j] = Hm[h, t*dh + j] -- the inverse of ``mix``."""
    B, H, Wm = Hm.shape
    if Wm % T:
        raise ValueError("mixed width must be divisible by T")
    dh = Wm // T
    out = np.empty((B, T, H * dh), dtype=Hm.dtype)
    for t in range(T):
        for h in range(H):
            out[:, t, h * dh:(h + 1) * dh] = Hm[:, h, t * dh:(t + 1) * dh]
    return out


# ---------------------------------------------------------------------------
# RMSNorm, Swish, SwiGLU   [TML] section 2.3.2-2.3.3, Eq. 17-18
# ---------------------------------------------------------------------------

def rmsnorm(v: np.ndarray, gamma: Optional[np.ndarray], eps: float) -> np.ndarray:
    """Llama-style RMSNorm over the last axis (no mean centring, [TML] 2.3.3;
    [TML-README] 'RMSNorm + no bias'): v / sqrt(mean(v^2) + eps) * gamma."""
    v = np.asarray(v, dtype=np.float64)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(ms + eps)
    out = v * r
    if gamma is not None:
        out = out * np.asarray(gamma, dtype=np.float64)
    return out


def silu(z: np.ndarray) -> np.ndarray:
    """Swish with beta = 1: z * sigmoid(z) ([TML] Eq. 17)."""
    z = np.asarray(z, dtype=np.float64)
    # sigmoid written in the branch that never overflows exp
    e = np.exp(-np.abs(z))
    sig = np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return z * sig


def softmax(l: np.ndarray) -> np.ndarray:
    l = np.asarray(l, dtype=np.float64)
    m = np.max(l, axis=-1, keepdims=True)
    e = np.exp(l - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def swiglu(v: np.ndarray, w_up: np.ndarray, w_gate: np.ndarray, w_down: np.ndarray,
           rho: bool = False) -> np.ndarray:
    """pSwiGLU of one position: FC_down(Swish(FC_gate(v)) * FC_up(v)) ([TML]
    Eq. 17-18), no bias, row-vector convention v @ W with W_up, W_gate [W, h]
    and W_down [h, W] ([RMX-GUIDE] 6.1: W1 [T, D, kD], W2 [T, kD, D]).
    In bf16 mode the hidden U is rounded to bf16 before the down projection."""
    v = np.asarray(v, dtype=np.float64)
    g = v @ np.asarray(w_gate, dtype=np.float64)
    u = v @ np.asarray(w_up, dtype=np.float64)
    U = _rho(silu(g) * u, rho)
    return U @ np.asarray(w_down, dtype=np.float64)


# ---------------------------------------------------------------------------
# FP8 serving   [TML] 2.5.2 (FP8 E4M3 post-training quantisation)
#
# The pages name the element format only. Reading: both operands of every
# GEMM are quantised, with microscaling -- one power-of-two scale per 32
# consecutive values along the contraction axis (the OCP MX layout: E4M3
# elements, E8M0 shared scales) -- fp32 accumulation, and bf16 activations
# between the GEMMs as in the bf16 path.
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0      # largest finite E4M3 value, 1.75 * 2**8
MX_BLOCK = 32


def e4m3_value(code) -> np.ndarray:
    """Value of FP8 E4M3 codes: sign bit, 4 exponent bits (bias 7), 3
    mantissa bits; exponent field 0 holds the subnormals m/8 * 2**-6; there
    are no infinities and S.1111.111 is NaN."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * mag)


_E4M3_NONNEG = e4m3_value(np.arange(0x7F))     # codes 0x00..0x7E, ascending 0 .. 448


def e4m3_round(x) -> np.ndarray:
    """E4M3 code of finite x: the nearest representable value, ties to the
    even code, with |x| > 448 taken as 448 (saturating conversion). The sign
    bit follows x (a negative value that rounds to zero gives 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.minimum(np.searchsorted(_E4M3_NONNEG, a, side="left"), 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_NONNEG[lo]
    d_hi = _E4M3_NONNEG[hi] - a
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def mx_exponent(amax) -> np.ndarray:
    """Shared exponent k of a block with largest magnitude amax: the block is
    stored as E4M3(x / 2**k) with k = floor(log2(amax)) - 8, 8 being the
    exponent of E4M3's largest normal, so the largest value maps into
    [2**8, 2**9) (values above 448 saturate). k is clamped to the E8M0 range
    [-127, 127]; an all-zero block takes -127."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)                       # amax = f * 2**e, 0.5 <= f < 1
    k = np.where(amax > 0, e - 1 - 8, -127)
    return np.clip(k, -127, 127).astype(np.int64)


def mx_quantize(x):
    """MXFP8 along the last axis (its length a multiple of 32): returns the
    E4M3 codes and the block exponents k. x is taken as fp32, the precision
    the quantised operands are produced in; x / 2**k is exact."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    n = x.shape[-1]
    if n % MX_BLOCK:
        raise ValueError(f"MX blocks need a multiple of {MX_BLOCK} values, got {n}")
    xb = x.reshape(x.shape[:-1] + (n // MX_BLOCK, MX_BLOCK))
    k = mx_exponent(np.max(np.abs(xb), axis=-1))
    codes = e4m3_round(np.ldexp(xb, -k[..., None]))
    return codes.reshape(x.shape), k


def mx_dequantize(codes, k) -> np.ndarray:
    codes = np.asarray(codes)
    n = codes.shape[-1]
    cb = codes.reshape(codes.shape[:-1] + (n // MX_BLOCK, MX_BLOCK))
    return (e4m3_value(cb) * np.exp2(np.asarray(k, np.float64))[..., None]).reshape(codes.shape)


def mx_round(x) -> np.ndarray:
    """Quantise to MXFP8 along the last axis and back (fp64 values)."""
    return mx_dequantize(*mx_quantize(x))


def swiglu_mx(v: np.ndarray, w_up: np.ndarray, w_gate: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """pSwiGLU of one position ([TML] Eq. 17-18) with MXFP8 GEMM operands
    ([TML] 2.5.2): the rows v and the columns of W_up, W_gate are quantised in
    blocks of 32 along W, the hidden U = silu(g) * u (fp32) and the columns of
    W_down in blocks of 32 along h; the products and sums are exact."""
    vq = mx_round(v)
    g = vq @ mx_round(np.asarray(w_gate).T).T
    u = vq @ mx_round(np.asarray(w_up).T).T
    U = mx_round(silu(g) * u)
    return U @ mx_round(np.asarray(w_down).T).T


# ---------------------------------------------------------------------------
# Sparse-Pertoken MoE   [TML] section 2.4, Eq. 19-21
# ---------------------------------------------------------------------------

def route(xhat: np.ndarray, w_router: np.ndarray, top_k: int, alpha: float):
    """Router of one position: logits l = xhat @ Wr, pi = softmax(l) over all
    E experts, chosen set = the top_k experts under the key (-l_e, e) (largest
    logit first, ties to the lowest index), gate = alpha * pi of the chosen
    experts, not renormalised ([TML] Eq. 19 and 21).

    Returns (idx [n, k] int, gate [n, k], logits [n, E], pi [n, E]).
    Output slots follow the same key order."""
    xhat = np.asarray(xhat, dtype=np.float64)
    logits = xhat @ np.asarray(w_router, dtype=np.float64)
    n, E = logits.shape
    if not 1 <= top_k <= E:
        raise ValueError("need 1 <= top_k <= E")
    pi = softmax(logits)
    experts = np.broadcast_to(np.arange(E), logits.shape)
    order = np.lexsort((experts, -logits), axis=-1)   # primary -l, then e
    idx = order[:, :top_k]
    gate = alpha * np.take_along_axis(pi, idx, axis=-1)
    return idx, gate, logits, pi


def moe(xhat: np.ndarray, w_router, exp_up, exp_gate, exp_down,
        sh_up, sh_gate, sh_down, top_k: int, alpha: float, rho: bool = False,
        idx_override: Optional[np.ndarray] = None, mx: bool = False):
    """Sparse-Pertoken MoE of one position ([TML] Eq. 19-21): the routed
    experts' SwiGLU outputs weighted by alpha * pi, plus the always-on shared
    SwiGLU expert of this position, ungated ([TML] 2.4.2). Only the chosen
    experts are evaluated, each on its own rows.

    ``idx_override`` [n, top_k] replaces the chosen set (gates stay alpha * pi
    of the named experts): where two logits sit closer than the rounding of
    the inputs can resolve, both top-k sets are correct results, and a
    comparison evaluates the method on the set the other side chose after
    checking that it is one of them.

    With ``mx`` the routed and shared experts' GEMMs take MXFP8 operands
    ([TML] 2.5.2 FP8 serving; swiglu_mx on the rows xhat); the router works on
    xhat itself, unquantised (the top-k choice depends on logit differences
    far below the fp8 step).

    Returns (y [n, W], idx, gate)."""
    idx, gate, _, pi = route(xhat, w_router, top_k, alpha)
    if idx_override is not None:
        idx = np.asarray(idx_override, dtype=np.int64).reshape(idx.shape)
        gate = alpha * np.take_along_axis(pi, idx, axis=-1)
    n = xhat.shape[0]
    E = np.asarray(w_router).shape[1]
    routed = np.zeros((n, np.asarray(exp_down).shape[-1]))
    for e in range(E):
        rows, slots = np.nonzero(idx == e)
        if rows.size == 0:
            continue
        if mx:
            ye = swiglu_mx(xhat[rows], exp_up[e], exp_gate[e], exp_down[e])
        else:
            ye = swiglu(xhat[rows], exp_up[e], exp_gate[e], exp_down[e], rho)
        routed[rows] += gate[rows, slots][:, None] * ye
    shared = swiglu_mx(xhat, sh_up, sh_gate, sh_down) if mx else swiglu(xhat, sh_up, sh_gate, sh_down, rho)
    return routed + shared, idx, gate


# ---------------------------------------------------------------------------
# sub-layer, block, stack   [TML] Eq. 12 and 16 in Pre-Norm form,
# [TML-README] block diagram, [TML] 2.3.4 inter-residual
# ---------------------------------------------------------------------------

WeightGetter = Callable[[int, int, int, int], np.ndarray]

# weight kind ids (same numbering as the seeded generator and the C header)
_K_GAIN, _K_UP, _K_GATE, _K_DOWN = 0, 1, 2, 3
_K_ROUTER, _K_EUP, _K_EGATE, _K_EDOWN, _K_SUP, _K_SGATE, _K_SDOWN = 4, 5, 6, 7, 8, 9, 10


def sublayer_positions(x: np.ndarray, resid: np.ndarray, cfg, layer: int, sub: int,
                       weights: WeightGetter, extra: Optional[np.ndarray] = None,
                       rho: bool = False, record: Optional[dict] = None, mx: bool = False,
                       route_override: Optional[np.ndarray] = None,
                       positions: Optional[Sequence[int]] = None) -> np.ndarray:
    """One Pre-Norm sub-layer over position-major rows:
    out[:, p] = resid[:, p] + F_p(RMSNorm(x[:, p])) [+ extra[:, p]], rounded
    once in bf16 mode. x, resid, extra are [n, P, W]; F_p is the position's
    own SwiGLU (dense) or Sparse-Pertoken MoE. ``record`` (optional dict)
    receives per-position routing {(p): (idx, gate)} for MoE sub-layers.
    With ``mx`` the SwiGLU GEMMs run on MXFP8 operands (swiglu_mx): in a
    dense sub-layer on the fp32 normalised rows, in a MoE sub-layer on xhat
    as the bf16 path forms it (rounded to bf16 in bf16 mode: the router's
    input and the rows the expert kernels read). ``route_override``
    [n, P, top_k] (MoE only) names the chosen experts of every row and
    position (see ``moe``). ``positions`` (optional) evaluates only those
    positions; the others come back as NaN."""
    n, P, W = x.shape
    gain = weights(layer, sub, _K_GAIN, 0)
    F = np.zeros((n, P, W))
    if positions is not None:
        F[:, [p for p in range(P) if p not in set(positions)]] = np.nan
    for p in (range(P) if positions is None else positions):
        if mx and cfg.E == 0:
            F[:, p] = swiglu_mx(rmsnorm(x[:, p, :], gain, cfg.eps), weights(layer, sub, _K_UP, p),
                                weights(layer, sub, _K_GATE, p), weights(layer, sub, _K_DOWN, p))
            continue
        xh = _rho(rmsnorm(x[:, p, :], gain, cfg.eps), rho)
        if cfg.E == 0:
            F[:, p] = swiglu(xh, weights(layer, sub, _K_UP, p), weights(layer, sub, _K_GATE, p),
                             weights(layer, sub, _K_DOWN, p), rho)
        else:
            y, idx, gate = moe(xh, weights(layer, sub, _K_ROUTER, p),
                               weights(layer, sub, _K_EUP, p), weights(layer, sub, _K_EGATE, p),
                               weights(layer, sub, _K_EDOWN, p), weights(layer, sub, _K_SUP, p),
                               weights(layer, sub, _K_SGATE, p), weights(layer, sub, _K_SDOWN, p),
                               cfg.top_k, cfg.gate_scale, rho,
                               None if route_override is None else route_override[:, p], mx)
            F[:, p] = y
            if record is not None:
                record[p] = (idx, gate)
    out = np.asarray(resid, dtype=np.float64) + F
    if extra is not None:
        out = out + np.asarray(extra, dtype=np.float64)
    return _rho(out, rho)


def block_forward(X: np.ndarray, cfg, layer: int, weights: WeightGetter,
                  extra: Optional[np.ndarray] = None, rho: bool = False,
                  trace: Optional[dict] = None, mx: bool = False) -> np.ndarray:
    """One TokenMixer-Large block in Pre-Norm form ([TML-README] diagram;
    [TML] Eq. 12, 16 with Pre-Norm per section 2.3.3):
        Hm      = Mix(X)
        H_next  = Hm + F_mix(Norm(Hm))              (intra-mixing residual)
        X_rev   = Revert(H_next)
        X_next  = X + F_rev(Norm(X_rev)) [+ extra]  (residual to the block input)
    ``extra`` is the inter-residual term added before the single rounding."""
    Hm = mix(X, cfg.H)
    Hn = sublayer_positions(Hm, Hm, cfg, layer, 0, weights, None, rho,
                            None if trace is None else trace.setdefault((layer, 0), {}), mx)
    Xr = revert(Hn, cfg.T)
    if trace is not None:
        trace[("in", layer, 0)] = X
        trace[("in", layer, 1)] = Xr
    return sublayer_positions(Xr, X, cfg, layer, 1, weights, extra, rho,
                              None if trace is None else trace.setdefault((layer, 1), {}), mx)


def stack_forward(X: np.ndarray, cfg, weights: WeightGetter, rho: Optional[bool] = None,
                  trace: Optional[dict] = None, mx: Optional[bool] = None) -> np.ndarray:
    """The L-block stack with inter-residuals ([TML] 2.3.4; [TML-README]):
    Y_0 = X; Z_l = Block_l(Y_{l-1}); Y_l = Z_l + Y_{l-g} when g > 0,
    l mod g == 0 and l < L (never after the last block); else Y_l = Z_l.
    Returns Y_L. ``rho`` defaults to the workload's activations being bf16
    (dtype bf16 or mxfp8), ``mx`` to the dtype being mxfp8."""
    if mx is None:
        mx = cfg.dtype == "mxfp8"
    if rho is None:
        rho = cfg.dtype in ("bf16", "mxfp8")
    Y = [np.asarray(X, dtype=np.float64)]
    g = cfg.gap
    for l in range(1, cfg.L + 1):
        extra = Y[l - g] if (g > 0 and l % g == 0 and l < cfg.L) else None
        Y.append(block_forward(Y[l - 1], cfg, l, weights, extra, rho, trace, mx))
    return Y[cfg.L]


# ---------------------------------------------------------------------------
# closed forms of the work   [RMX-BOOK] 7.4.2 (Param = FLOPs = 2TkD^2 MACs)
# ---------------------------------------------------------------------------

def param_count_closed_form(cfg) -> int:
    """Weights of the stack: dense L * sum_sub 3 P W h; MoE
    L * sum_sub P (3 E W h_e + 3 W h_s + W E). Norm gains excluded."""
    total = 0
    for sub in (0, 1):
        P = cfg.H if sub == 0 else cfg.T
        W = cfg.T * cfg.D // cfg.H if sub == 0 else cfg.D
        if cfg.E == 0:
            h = cfg.hidden_mix if sub == 0 else cfg.hidden_rev
            total += 3 * P * W * h
        else:
            total += P * (3 * cfg.E * W * cfg.expert_hidden + 3 * W * cfg.shared_hidden + W * cfg.E)
    return cfg.L * total


def flops_per_sample(cfg) -> int:
    """Algorithmic GEMM FLOPs (2 per multiply-add) of one sample's forward:
    up, gate and down of every position; for MoE only the k chosen experts,
    the shared expert and the router count."""
    total = 0
    for sub in (0, 1):
        P = cfg.H if sub == 0 else cfg.T
        W = cfg.T * cfg.D // cfg.H if sub == 0 else cfg.D
        if cfg.E == 0:
            h = cfg.hidden_mix if sub == 0 else cfg.hidden_rev
            total += 2 * P * 3 * W * h
        else:
            total += 2 * P * (3 * cfg.top_k * W * cfg.expert_hidden
                              + 3 * W * cfg.shared_hidden + W * cfg.E)
    return cfg.L * total


# ---------------------------------------------------------------------------
# RankMixer block   [RMX-BOOK] 7.4.0 block equations, 7.4.1, 7.4.2;
# [RMX-GUIDE] sections 5, 6.1 and 7; the RankMixer README's per-token FFN
#
# Readings (the pages leave these open):
# * LN is LayerNorm over the token width: subtract the row mean, divide by
#   sqrt(biased variance + eps), then gain and bias ([RMX-GUIDE] 7 names the
#   residual + LN of the block; the chapter's block equations use LN).
# * GELU is the exact form z * Phi(z) with Phi the standard normal CDF (the
#   pages write GELU without an approximation).
# * Post-LN as the chapter's block equations write it ([RMX-GUIDE] 7 allows
#   pre or post; the equations fix post).
# * bf16 precision contract, as for TokenMixer-Large: inputs, weights,
#   biases and norm parameters are bf16 values; S (the FFN input and its
#   residual), the hidden GELU output and the block output are rounded to
#   bf16 once each; LN statistics, the GEMM accumulations, the biases' and
#   residual's additions stay unrounded.
# * Sparse version ([RMX-BOOK] 7.4.3, inference router): each token's
#   experts have the per-token FFN's form (GELU, biases); the router is a
#   bias-free linear map; the gate multiplies the expert's whole output,
#   its second bias included; in bf16 mode the gated hidden is the rounded
#   quantity and the gates themselves are not rounded.
# ---------------------------------------------------------------------------

_K_NBIAS, _K_BUP, _K_BDOWN = 11, 12, 13
_K_EBUP, _K_EBDOWN = 14, 15


def layernorm(v: np.ndarray, gamma: Optional[np.ndarray], beta: Optional[np.ndarray],
              eps: float) -> np.ndarray:
    """LayerNorm over the last axis: (v - mean) / sqrt(var + eps) * gamma + beta,
    var the biased (1/n) variance."""
    v = np.asarray(v, dtype=np.float64)
    mu = np.mean(v, axis=-1, keepdims=True)
    d = v - mu
    var = np.mean(d * d, axis=-1, keepdims=True)
    out = d / np.sqrt(var + eps)
    if gamma is not None:
        out = out * np.asarray(gamma, dtype=np.float64)
    if beta is not None:
        out = out + np.asarray(beta, dtype=np.float64)
    return out


def gelu(z: np.ndarray) -> np.ndarray:
    """Exact GELU: z * Phi(z), Phi(z) = (1 + erf(z / sqrt 2)) / 2."""
    z = np.asarray(z, dtype=np.float64)
    erf = np.vectorize(math.erf, otypes=[np.float64])
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def pffn(s: np.ndarray, w1: np.ndarray, b1: np.ndarray, w2: np.ndarray, b2: np.ndarray,
         rho: bool = False) -> np.ndarray:
    """One token's own FFN ([RMX-BOOK] 7.4.2; the RankMixer README's per-token
    FFN): v = GELU(s W1 + b1) W2 + b2, row-vector convention with W1 [D, kD],
    W2 [kD, D] ([RMX-GUIDE] 6.1). In bf16 mode the hidden is rounded to bf16
    before the second matrix."""
    s = np.asarray(s, dtype=np.float64)
    hid = _rho(gelu(s @ np.asarray(w1, dtype=np.float64) + np.asarray(b1, dtype=np.float64)), rho)
    return hid @ np.asarray(w2, dtype=np.float64) + np.asarray(b2, dtype=np.float64)


def rankmixer_block(X: np.ndarray, cfg, layer: int, weights: WeightGetter,
                    rho: bool = False, trace: Optional[dict] = None) -> np.ndarray:
    """One RankMixer block ([RMX-BOOK] 7.4.0):
        S      = LN_1(TokenMixing(X) + X)
        X_next = LN_2(PFFN(S) + S)
    TokenMixing is the parameter-free head split and cross-token concat
    ([RMX-BOOK] 7.4.1) with H = T ([RMX-GUIDE] 5), so its output has the
    shape of X and the residual adds token by token. PFFN applies token t's
    own FFN to S[:, t]. LN_1 belongs to sub-layer 0, the FFN and LN_2 to
    sub-layer 1. ``trace`` (optional dict) receives S under (layer, 'S')."""
    B, T, D = X.shape
    if cfg.H != T:
        raise ValueError("RankMixer token mixing needs H == T")
    X = np.asarray(X, dtype=np.float64)
    S = _rho(layernorm(mix(X, cfg.H) + X, weights(layer, 0, _K_GAIN, 0),
                       weights(layer, 0, _K_NBIAS, 0), cfg.eps), rho)
    if trace is not None:
        trace[(layer, "S")] = S
    return rankmixer_ffn_sublayer(S, cfg, layer, weights, rho)


def relu_route(s: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """ReLU routing ([RMX-BOOK] 7.4.3; the RankMixer README's ReLU routing):
    G = ReLU(h(s)) with h the token's linear inference router s @ Wr, Wr
    [D, E], no bias. A gate of 0 leaves its expert inactive, so each row
    activates its own number of experts."""
    return np.maximum(np.asarray(s, dtype=np.float64) @ np.asarray(w_router, dtype=np.float64), 0.0)


def relu_moe(s: np.ndarray, w_router, w1, b1, w2, b2, rho: bool = False):
    """v = sum_j G_j e_j(s) ([RMX-BOOK] 7.4.3) over one token's E experts,
    each e_j the per-token FFN's form GELU(s W1_j + b1_j) W2_j + b2_j with
    W1 [E, D, h_e], b1 [E, h_e], W2 [E, h_e, D], b2 [E, D]. In bf16 mode the
    gated hidden G_j * GELU(.) is rounded once before the second matrix.
    Returns (v, G)."""
    s = np.asarray(s, dtype=np.float64)
    G = relu_route(s, w_router)
    v = np.zeros((s.shape[0], np.asarray(w2).shape[-1]))
    for j in range(G.shape[1]):
        g = G[:, j:j + 1]
        hid = _rho(g * gelu(s @ np.asarray(w1[j], dtype=np.float64) + np.asarray(b1[j], dtype=np.float64)), rho)
        v += hid @ np.asarray(w2[j], dtype=np.float64) + g * np.asarray(b2[j], dtype=np.float64)
    return v, G


def rankmixer_ffn_sublayer(S: np.ndarray, cfg, layer: int, weights: WeightGetter,
                           rho: bool = False, record: Optional[dict] = None) -> np.ndarray:
    """Second half of a RankMixer block: X_next[:, t] = LN_2(S[:, t] + F_t(S[:, t])),
    F_t the token's FFN (dense) or its ReLU-routed experts (E > 0; the
    gates of token t go to ``record[t]``)."""
    S = np.asarray(S, dtype=np.float64)
    out = np.empty_like(S)
    g2, b2n = weights(layer, 1, _K_GAIN, 0), weights(layer, 1, _K_NBIAS, 0)
    for t in range(S.shape[1]):
        if cfg.E == 0:
            v = pffn(S[:, t], weights(layer, 1, _K_UP, t), weights(layer, 1, _K_BUP, t),
                     weights(layer, 1, _K_DOWN, t), weights(layer, 1, _K_BDOWN, t), rho)
        else:
            v, G = relu_moe(S[:, t], weights(layer, 1, _K_ROUTER, t), weights(layer, 1, _K_EUP, t),
                            weights(layer, 1, _K_EBUP, t), weights(layer, 1, _K_EDOWN, t),
                            weights(layer, 1, _K_EBDOWN, t), rho)
            if record is not None:
                record[t] = G
        out[:, t] = layernorm(S[:, t] + v, g2, b2n, cfg.eps)
    return _rho(out, rho)


def rankmixer_stack(X: np.ndarray, cfg, weights: WeightGetter, rho: Optional[bool] = None,
                    trace: Optional[dict] = None) -> np.ndarray:
    """L stacked RankMixer blocks ([RMX-BOOK] 7.4.0: X_n from X_{n-1}); no
    inter-residual. ``rho`` defaults to the workload being bf16."""
    if rho is None:
        rho = cfg.dtype == "bf16"
    Y = np.asarray(X, dtype=np.float64)
    for l in range(1, cfg.L + 1):
        Y = rankmixer_block(Y, cfg, l, weights, rho, trace)
    return Y


def rankmixer_flops_per_sample(cfg) -> int:
    """GEMM FLOPs of one sample: per block and token 2 * (D kD + kD D)
    ([RMX-BOOK] 7.4.2: 2TkD^2 multiply-adds per block). For the ReLU-routed
    experts, every expert of the token and the router (what a forward that
    evaluates each expert on all rows computes; rows with a zero gate need
    none of it)."""
    if cfg.E == 0:
        return cfg.L * cfg.T * 2 * 2 * cfg.D * cfg.hidden_rev
    return cfg.L * cfg.T * 2 * (2 * cfg.D * cfg.E * cfg.expert_hidden + cfg.D * cfg.E)


# ---------------------------------------------------------------------------
# Model front and back   [TML] 2.2 Eq. 1-4 (semantic group-wise tokenizer,
# global token), [TML] 2.1 (mean pooling of the output tokens for the
# prediction), [TML-README] block diagram (group MLPs + global MLP -> tokens;
# mean-pool over tokens -> projection head -> logit)
#
# Readings (the pages name the MLPs but not their form):
# * every MLP here (MLP_i of a group, MLP_g of the global token, the
#   projection head) is two bias-free linear maps with ReLU between them,
#   v -> ReLU(v W1) W2 (bias off as everywhere in the model, [TML-README]);
# * the tokenizer's input is the embeddings e of Eq. 1 already concatenated
#   group by group, [n, F], F = sum of the T - 1 group widths; group t
#   (1 <= t < T) is columns [off_t, off_t + d_t); the global token reads all
#   F columns (Eq. 3) and is position 0 (Eq. 4);
# * the head averages the T output tokens, applies its MLP and returns one
#   logit per sample (one task; no sigmoid -- the pages end at the logit);
# * bf16 contract as in the stack: the hidden ReLU outputs, the tokens X
#   and the pooled mean are rounded to bf16 once each; sums and the logit
#   stay unrounded.
# ---------------------------------------------------------------------------

_K_TOK_UP, _K_TOK_DOWN, _K_HEAD_UP, _K_HEAD_DOWN = 16, 17, 18, 19


def relu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return np.where(z > 0, z, 0.0)


def mlp2(v: np.ndarray, w1: np.ndarray, w2: np.ndarray, rho: bool = False) -> np.ndarray:
    """ReLU(v W1) W2, no biases; in bf16 mode the hidden is rounded once."""
    h = _rho(relu(np.asarray(v, dtype=np.float64) @ np.asarray(w1, dtype=np.float64)), rho)
    return h @ np.asarray(w2, dtype=np.float64)


def group_offsets(group_widths) -> np.ndarray:
    """Column offset of each semantic group in the concatenated embeddings."""
    return np.concatenate([[0], np.cumsum(np.asarray(group_widths, dtype=np.int64))])


def tokenize(emb: np.ndarray, cfg, weights: WeightGetter, rho: bool = False) -> np.ndarray:
    """[TML] Eq. 2-4: X_t = MLP_t(group t's embeddings) for t = 1..T-1, the
    global token X_0 = MLP_g(all F columns). emb [n, F] -> X [n, T, D]."""
    emb = np.asarray(emb, dtype=np.float64)
    off = group_offsets(cfg.groups)
    if len(cfg.groups) != cfg.T - 1 or emb.shape[1] != off[-1]:
        raise ValueError("need T - 1 groups whose widths sum to the embedding width")
    X = np.empty((emb.shape[0], cfg.T, cfg.D))
    for t in range(cfg.T):
        v = emb if t == 0 else emb[:, off[t - 1]:off[t]]
        X[:, t] = mlp2(v, weights(0, 0, _K_TOK_UP, t), weights(0, 0, _K_TOK_DOWN, t), rho)
    return _rho(X, rho)


def head(Y: np.ndarray, cfg, weights: WeightGetter, rho: bool = False) -> np.ndarray:
    """[TML] 2.1, [TML-README]: mean over the T output tokens, then the
    projection MLP to one logit per sample. Y [n, T, D] -> logits [n]."""
    pooled = _rho(np.mean(np.asarray(Y, dtype=np.float64), axis=1), rho)
    w2 = np.asarray(weights(0, 0, _K_HEAD_DOWN, 0), dtype=np.float64).reshape(-1, 1)
    return mlp2(pooled, weights(0, 0, _K_HEAD_UP, 0), w2, rho)[:, 0]


def model_forward(emb: np.ndarray, cfg, weights: WeightGetter, rho: Optional[bool] = None) -> np.ndarray:
    """Embeddings -> tokens -> the block stack -> mean-pool head -> logits."""
    if rho is None:
        rho = cfg.dtype in ("bf16", "mxfp8")
    X = tokenize(emb, cfg, weights, rho)
    Y = rankmixer_stack(X, cfg, weights, rho) if cfg.rankmixer else stack_forward(X, cfg, weights, rho)
    return head(Y, cfg, weights, rho)


def io_flops_per_sample(cfg) -> int:
    """GEMM FLOPs of the tokenizer and the head for one sample."""
    F = int(np.sum(cfg.groups))
    tok = 2 * (2 * F * cfg.tok_hidden + cfg.T * cfg.tok_hidden * cfg.D)
    return tok + 2 * (cfg.D * cfg.head_hidden + cfg.head_hidden)

"""Seeded synthetic inputs for the TokenMixer-Large block stack.

This module is shared by the CPU oracle and by the GPU tests/bench. It holds
the workload descriptions and the random draws only: none of the method's
arithmetic lives here.

Draws follow one recipe everywhere:

* ``numpy.random.Generator(PCG64(SeedSequence(seed, spawn_key=key)))`` and
  ``standard_normal(dtype=float32)``;
* key ``(0,)`` for the token tensor X, key ``(1, layer, sub, kind, position)``
  for one position's slice of a weight bank, so every slice can be regenerated
  on its own, in any order, in parallel;
* token values are N(0, 1); up / gate / router weights N(0, 1/fan_in) with
  fan_in the input width W; every down matrix 0.01 * N(0, 1/fan_in) with
  fan_in its hidden size (the pages' down-matrix small init, TokenMixer-Large
  summary section 2.4.4, realised with the normal init the workloads state);
* for bf16 workloads every draw is rounded to the nearest bf16 value
  (ties to even) by torch's fp32 -> bf16 conversion, so both sides consume
  the very same bf16-representable numbers.
"""
from __future__ import annotations

import dataclasses
import os
from typing import Dict, Optional, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

SUB_MIX = 0
SUB_REVERT = 1

# weight kinds (values match the C header's TMX_W_* enumerators)
K_NORM_GAIN = 0
K_UP = 1
K_GATE = 2
K_DOWN = 3
K_ROUTER = 4
K_EXP_UP = 5
K_EXP_GATE = 6
K_EXP_DOWN = 7
K_SH_UP = 8
K_SH_GATE = 9
K_SH_DOWN = 10
K_NORM_BIAS = 11     # RankMixer LayerNorm bias
K_BIAS_UP = 12       # RankMixer per-token FFN first bias  [P, h]
K_BIAS_DOWN = 13     # RankMixer per-token FFN second bias [P, W]
K_EXP_BIAS_UP = 14   # RankMixer ReLU-routed experts' first biases  [P, E, h_e]
K_EXP_BIAS_DOWN = 15 # RankMixer ReLU-routed experts' second biases [P, E, W]
# model front and back (one bank each, not per layer): the tokenizer's first
# layers [2F, h_tok] (the global token's [F, h_tok], then every group's
# [d_t, h_tok] in group order), second layers [T, h_tok, D], the head's
# [D, h_head] and [h_head]
K_TOK_UP = 16
K_TOK_DOWN = 17
K_HEAD_UP = 18
K_HEAD_DOWN = 19
IO_KINDS = (K_TOK_UP, K_TOK_DOWN, K_HEAD_UP, K_HEAD_DOWN)

KIND_NAMES = {
    K_NORM_GAIN: "norm_gain", K_UP: "up", K_GATE: "gate", K_DOWN: "down",
    K_ROUTER: "router", K_EXP_UP: "exp_up", K_EXP_GATE: "exp_gate",
    K_EXP_DOWN: "exp_down", K_SH_UP: "sh_up", K_SH_GATE: "sh_gate",
    K_SH_DOWN: "sh_down", K_NORM_BIAS: "norm_bias", K_BIAS_UP: "bias_up",
    K_BIAS_DOWN: "bias_down", K_EXP_BIAS_UP: "exp_bias_up", K_EXP_BIAS_DOWN: "exp_bias_down",
    K_TOK_UP: "tok_up", K_TOK_DOWN: "tok_down", K_HEAD_UP: "head_up", K_HEAD_DOWN: "head_down",
}

DENSE_KINDS = (K_UP, K_GATE, K_DOWN)
DOWN_KINDS = (K_DOWN, K_EXP_DOWN, K_SH_DOWN)   # the kinds that carry the small-down factor
MOE_KINDS = (K_ROUTER, K_EXP_UP, K_EXP_GATE, K_EXP_DOWN, K_SH_UP, K_SH_GATE, K_SH_DOWN)
# RankMixer: the token-mixing sub-layer has only its LayerNorm; the per-token
# FFN sub-layer holds W1 (K_UP), W2 (K_DOWN) and their biases
RMX_FFN_KINDS = (K_UP, K_DOWN, K_BIAS_UP, K_BIAS_DOWN)
# RankMixer sparse MoE (ReLU routing, inference router): router, the
# experts' two matrices and their biases
RMX_MOE_KINDS = (K_ROUTER, K_EXP_UP, K_EXP_DOWN, K_EXP_BIAS_UP, K_EXP_BIAS_DOWN)
NORM_KINDS = (K_NORM_GAIN, K_NORM_BIAS)

BLOCK_TML = "tml"
BLOCK_RANKMIXER = "rankmixer"


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and init of one block-stack workload."""
    name: str
    B: int
    T: int
    H: int
    D: int
    L: int
    hidden_mix: int = 0      # dense per-token hidden of the mix sub-layer
    hidden_rev: int = 0      # dense per-token hidden of the revert sub-layer
    E: int = 0               # routed experts per position (0 = dense)
    top_k: int = 0
    expert_hidden: int = 0
    shared_hidden: int = 0
    alpha: float = 0.0       # 0 means E / top_k
    eps: float = 1e-6
    gap: int = 2             # inter-residual gap (0 = none)
    dtype: str = "bf16"      # "bf16", "f32", or "mxfp8" (bf16 activations and weights,
                             # MXFP8 GEMM operands inside the library)
    seed: int = 0
    down_scale: float = 0.01
    block: str = BLOCK_TML   # "tml" (TokenMixer-Large) or "rankmixer"
    random_norm: bool = False  # draw LayerNorm gains / biases instead of 1 / 0
    groups: Tuple[int, ...] = ()   # model front: widths of the T - 1 semantic groups
    tok_hidden: int = 0        # hidden width of the tokenizer MLPs
    head_hidden: int = 0       # hidden width of the projection head

    # -- derived -----------------------------------------------------------
    @property
    def moe(self) -> bool:
        return self.E > 0

    @property
    def bf16_values(self) -> bool:
        """Activations and weights are handed over as bf16 values."""
        return self.dtype in ("bf16", "mxfp8")

    @property
    def dh(self) -> int:
        return self.D // self.H

    @property
    def gate_scale(self) -> float:
        return self.alpha if self.alpha != 0.0 else self.E / self.top_k

    def positions(self, sub: int) -> int:
        return self.H if sub == SUB_MIX else self.T

    def width(self, sub: int) -> int:
        return self.T * self.D // self.H if sub == SUB_MIX else self.D

    def hidden(self, sub: int) -> int:
        return self.hidden_mix if sub == SUB_MIX else self.hidden_rev

    @property
    def rankmixer(self) -> bool:
        return self.block == BLOCK_RANKMIXER

    def kinds(self):
        return MOE_KINDS if self.moe else DENSE_KINDS

    def sub_kinds(self, sub: int):
        """Matrix and bias kinds of one sub-layer (norm parameters excluded)."""
        if self.rankmixer:
            if sub != SUB_REVERT:
                return ()
            return RMX_MOE_KINDS if self.moe else RMX_FFN_KINDS
        return self.kinds()

    def kind_shape(self, sub: int, kind: int) -> Tuple[int, ...]:
        """Logical row-major shape of one (sub-layer, kind) bank, all positions."""
        P, W = self.positions(sub), self.width(sub)
        if kind in NORM_KINDS:
            return (W,)
        if kind == K_BIAS_UP:
            return (P, self.hidden(sub))
        if kind == K_BIAS_DOWN:
            return (P, W)
        if kind == K_EXP_BIAS_UP:
            return (P, self.E, self.expert_hidden)
        if kind == K_EXP_BIAS_DOWN:
            return (P, self.E, W)
        if kind in (K_UP, K_GATE):
            return (P, W, self.hidden(sub))
        if kind == K_DOWN:
            return (P, self.hidden(sub), W)
        if kind == K_ROUTER:
            return (P, W, self.E)
        if kind in (K_EXP_UP, K_EXP_GATE):
            return (P, self.E, W, self.expert_hidden)
        if kind == K_EXP_DOWN:
            return (P, self.E, self.expert_hidden, W)
        if kind in (K_SH_UP, K_SH_GATE):
            return (P, W, self.shared_hidden)
        if kind == K_SH_DOWN:
            return (P, self.shared_hidden, W)
        raise ValueError(f"unknown kind {kind}")

    def fan_in(self, sub: int, kind: int) -> int:
        if kind in (K_DOWN, K_BIAS_DOWN):
            return self.hidden(sub)
        if kind in (K_EXP_DOWN, K_EXP_BIAS_DOWN):
            return self.expert_hidden
        if kind == K_SH_DOWN:
            return self.shared_hidden
        return self.width(sub)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def has_io(self) -> bool:
        """The workload includes the tokenizer front and the mean-pool head."""
        return len(self.groups) > 0

    @property
    def emb_width(self) -> int:
        return int(sum(self.groups))

    def io_shape(self, kind: int) -> Tuple[int, ...]:
        F, h, hh = self.emb_width, self.tok_hidden, self.head_hidden
        return {K_TOK_UP: (2 * F, h), K_TOK_DOWN: (self.T, h, self.D), K_HEAD_UP: (self.D, hh),
                K_HEAD_DOWN: (hh,)}[kind]

    def io_rows(self, kind: int, t: int) -> Tuple[int, int]:
        """Row range of position t's slice of a tokenizer bank."""
        F = self.emb_width
        if kind == K_TOK_UP:
            if t == 0:
                return 0, F
            off = int(sum(self.groups[:t - 1]))
            return F + off, F + off + self.groups[t - 1]
        return t, t + 1


# The five workloads of the block-stack forward (TokenMixer-Large summary,
# sections 2.3-2.4; batch sizes as in the reproduction README's commands).
WORKLOADS: Dict[int, Workload] = {
    1: Workload("tiny_dense_fp32", B=128, T=4, H=4, D=32, L=1, hidden_mix=64,
                hidden_rev=64, gap=2, dtype="f32", seed=0),
    2: Workload("dense_pertoken_swiglu", B=4096, T=16, H=16, D=256, L=4,
                hidden_mix=1024, hidden_rev=1024, gap=2, seed=1),
    3: Workload("uneven_mixing_h8", B=4096, T=16, H=8, D=256, L=4,
                hidden_mix=1024, hidden_rev=1024, gap=2, seed=2),
    4: Workload("sparse_pertoken_moe", B=4096, T=16, H=16, D=512, L=8, E=16,
                top_k=4, expert_hidden=256, shared_hidden=512, alpha=4.0,
                gap=2, seed=3),
    5: Workload("large_moe_15b", B=8192, T=32, H=32, D=768, L=8, E=32,
                top_k=4, expert_hidden=384, shared_hidden=768, alpha=8.0,
                gap=2, seed=4),
}


# Whole-model workloads: the tokenizer front (T - 1 semantic groups of mixed
# widths, a global token) and the mean-pool head around a block stack
def _mixed_groups(n, widths):
    return tuple(widths[i % len(widths)] for i in range(n))


MODEL_WORKLOADS: Dict[str, Workload] = {
    "model_dense": WORKLOADS[2].with_(name="model_dense", groups=_mixed_groups(15, (128, 256, 384)),
                                      tok_hidden=256, head_hidden=256, seed=21),
    "model_moe_15b": WORKLOADS[5].with_(name="model_moe_15b", groups=_mixed_groups(31, (128, 256, 384)),
                                        tok_hidden=768, head_hidden=256, seed=24),
}


# RankMixer block stacks (the fun-rec chapter 7.4.0 block equations, H = T
# as the reproduction guide's section 5 requires; per-token FFN hidden
# kD = 4D as the guide's W1 [T, D, kD] with k = 4). Standard N(0, 1/fan_in)
# init for both FFN matrices (post-LN blocks have no small-down init) and
# LayerNorm eps 1e-5.
RANKMIXER_WORKLOADS: Dict[str, Workload] = {
    "rankmixer_d256": Workload("rankmixer_d256", B=4096, T=16, H=16, D=256, L=4,
                               hidden_rev=1024, gap=0, eps=1e-5, seed=11,
                               down_scale=1.0, block=BLOCK_RANKMIXER),
    "rankmixer_d512": Workload("rankmixer_d512", B=4096, T=16, H=16, D=512, L=4,
                               hidden_rev=2048, gap=0, eps=1e-5, seed=12,
                               down_scale=1.0, block=BLOCK_RANKMIXER),
    # sparse version: every token's FFN replaced by 16 ReLU-routed experts of
    # hidden 128 (fun-rec chapter 7.4.3 ReLU routing, inference router)
    "rankmixer_moe_d256": Workload("rankmixer_moe_d256", B=4096, T=16, H=16, D=256, L=4,
                                   E=16, expert_hidden=128, gap=0, eps=1e-5, seed=13,
                                   down_scale=1.0, block=BLOCK_RANKMIXER),
}


# ---------------------------------------------------------------------------
# draws
# ---------------------------------------------------------------------------

def _rng(seed: int, key: Tuple[int, ...]) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def to_bf16_values(a: np.ndarray) -> np.ndarray:
    """Nearest bf16 values (ties to even) of an fp32 array, returned as fp32."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Bit patterns of the nearest bf16 values (ties to even) of finite fp32
    data: input quantisation for bulk generation (a CPU test checks it equals
    torch's fp32 -> bf16 conversion)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _finish(cfg: Workload, a: np.ndarray) -> np.ndarray:
    return to_bf16_values(a) if cfg.bf16_values else a


def make_x(cfg: Workload, seed: Optional[int] = None, B: Optional[int] = None) -> np.ndarray:
    """Token tensor X [B, T, D], N(0, 1) (fp32 array of dtype-representable values)."""
    s = cfg.seed if seed is None else seed
    n = cfg.B if B is None else B
    a = _rng(s, (0,)).standard_normal((n, cfg.T, cfg.D), dtype=np.float32)
    return _finish(cfg, a)


def _draw(cfg: Workload, layer: int, sub: int, kind: int, p: int, seed: Optional[int]) -> np.ndarray:
    """Unrounded fp32 draw of one position's slice: N(0, 1/fan_in), downs x0.01."""
    shape = cfg.kind_shape(sub, kind)
    s = cfg.seed if seed is None else seed
    a = _rng(s, (1, layer, sub, kind, p)).standard_normal(shape[1:], dtype=np.float32)
    std = np.float32(1.0 / np.sqrt(cfg.fan_in(sub, kind)))
    if kind in (K_DOWN, K_EXP_DOWN, K_SH_DOWN):
        std = np.float32(std * cfg.down_scale)
    a *= std
    return a


def make_emb(cfg: Workload, seed: Optional[int] = None, B: Optional[int] = None) -> np.ndarray:
    """Concatenated feature embeddings [B, F] (the tokenizer's input), N(0, 1)."""
    s = cfg.seed if seed is None else seed
    n = cfg.B if B is None else B
    a = _rng(s, (3,)).standard_normal((n, cfg.emb_width), dtype=np.float32)
    return _finish(cfg, a)


def io_slice(cfg: Workload, kind: int, t: int = 0, seed: Optional[int] = None) -> np.ndarray:
    """Position t's slice of a tokenizer / head bank, N(0, 1/fan_in), drawn
    under key (2, kind, t); fp32 array of dtype-representable values."""
    s = cfg.seed if seed is None else seed
    if kind == K_TOK_UP:
        lo, hi = cfg.io_rows(kind, t)
        shape, fan = (hi - lo, cfg.tok_hidden), hi - lo
    elif kind == K_TOK_DOWN:
        shape, fan = (cfg.tok_hidden, cfg.D), cfg.tok_hidden
    elif kind == K_HEAD_UP:
        shape, fan = (cfg.D, cfg.head_hidden), cfg.D
    else:
        shape, fan = (cfg.head_hidden,), cfg.head_hidden
    a = _rng(s, (2, kind, t)).standard_normal(shape, dtype=np.float32) * np.float32(1.0 / np.sqrt(fan))
    return _finish(cfg, a)


def io_banks(cfg: Workload, seed: Optional[int] = None):
    """{(0, 0, kind): bank} of the tokenizer and the head, in the library's
    layouts (bf16 bit patterns for bf16 workloads)."""
    out = {}
    for kind in IO_KINDS:
        if kind == K_TOK_UP:
            a = np.concatenate([io_slice(cfg, kind, t, seed) for t in range(cfg.T)], axis=0)
        elif kind == K_TOK_DOWN:
            a = np.stack([io_slice(cfg, kind, t, seed) for t in range(cfg.T)])
        else:
            a = io_slice(cfg, kind, 0, seed)
        out[(0, 0, kind)] = f32_to_bf16_bits(a) if cfg.bf16_values else a
    return out


def _norm_param(cfg: Workload, layer: int, sub: int, kind: int, seed: Optional[int]) -> np.ndarray:
    """Norm gain (1) or bias (0); with ``random_norm`` gain 1 + 0.1 N(0, 1) and
    bias 0.1 N(0, 1), drawn under the weight key of position 0."""
    W = cfg.width(sub)
    if not cfg.random_norm:
        return (np.ones if kind == K_NORM_GAIN else np.zeros)(W, np.float32)
    s = cfg.seed if seed is None else seed
    a = _rng(s, (1, layer, sub, kind, 0)).standard_normal(W, dtype=np.float32) * np.float32(0.1)
    if kind == K_NORM_GAIN:
        a += np.float32(1.0)
    return _finish(cfg, a)


def weight_slice(cfg: Workload, layer: int, sub: int, kind: int, p: int,
                 seed: Optional[int] = None) -> np.ndarray:
    """One position's slice of a weight bank (fp32 array, dtype-representable)."""
    if kind in NORM_KINDS:
        return _norm_param(cfg, layer, sub, kind, seed)
    return _finish(cfg, _draw(cfg, layer, sub, kind, p, seed))


def weight_bank(cfg: Workload, layer: int, sub: int, kind: int,
                seed: Optional[int] = None) -> np.ndarray:
    """A whole (layer, sub-layer, kind) bank, all positions stacked (fp32 values)."""
    if kind in NORM_KINDS:
        return weight_slice(cfg, layer, sub, kind, 0, seed)
    return np.stack([weight_slice(cfg, layer, sub, kind, p, seed) for p in range(cfg.positions(sub))])


def default_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def weight_banks(cfg: Workload, seed: Optional[int] = None, workers: int = 0, kinds=None):
    """{(layer 1..L, sub, kind): bank} for every matrix bank of the stack
    (only the kinds in ``kinds`` when it is given).

    bf16 workloads give uint16 arrays of bf16 bit patterns, fp32 workloads
    float32 arrays. Slices are drawn in a thread pool (the generator releases
    the GIL); every slice has its own seed key, so the values do not depend
    on ``workers`` -- nor on which other kinds are drawn: two workloads that
    differ only in ``down_scale`` share every bank but the down matrices."""
    from concurrent.futures import ThreadPoolExecutor
    bf16 = cfg.bf16_values
    banks = {}
    jobs = []
    for l in range(1, cfg.L + 1):
        for s in (SUB_MIX, SUB_REVERT):
            if cfg.random_norm:
                for k in NORM_KINDS if cfg.rankmixer else (K_NORM_GAIN,):
                    if kinds is not None and k not in kinds:
                        continue
                    v = _norm_param(cfg, l, s, k, seed)
                    banks[(l, s, k)] = f32_to_bf16_bits(v) if bf16 else v
            for k in cfg.sub_kinds(s):
                if kinds is not None and k not in kinds:
                    continue
                shape = cfg.kind_shape(s, k)
                arr = np.empty(shape, np.uint16 if bf16 else np.float32)
                banks[(l, s, k)] = arr
                jobs.extend((arr, l, s, k, p) for p in range(shape[0]))

    def run(job):
        arr, l, s, k, p = job
        a = _draw(cfg, l, s, k, p, seed)
        arr[p] = f32_to_bf16_bits(a) if bf16 else a

    n = workers or default_workers()
    if n > 1:
        with ThreadPoolExecutor(max_workers=n) as ex:
            list(ex.map(run, jobs))
    else:
        for j in jobs:
            run(j)
    return banks


def param_count(cfg: Workload) -> int:
    """Number of weight and bias values of the stack (norm parameters excluded)."""
    total = 0
    for sub in (SUB_MIX, SUB_REVERT):
        for kind in cfg.sub_kinds(sub):
            total += int(np.prod(cfg.kind_shape(sub, kind)))
    return total * cfg.L


class WeightSource:
    """Lazy (layer 1..L, sub, kind, position) -> fp32 slice. With ``banks``
    (from :func:`weight_banks`) slices are decoded from them, else drawn."""

    def __init__(self, cfg: Workload, banks=None, seed: Optional[int] = None):
        self.cfg = cfg
        self.banks = banks
        self.seed = seed

    def __call__(self, layer: int, sub: int, kind: int, p: int) -> np.ndarray:
        if kind in IO_KINDS:
            if self.banks is not None and (0, 0, kind) in self.banks:
                b = self.banks[(0, 0, kind)]
                if kind == K_TOK_UP:
                    lo, hi = self.cfg.io_rows(kind, p)
                    b = b[lo:hi]
                elif kind == K_TOK_DOWN:
                    b = b[p]
                return bf16_bits_to_f32(b) if b.dtype == np.uint16 else b
            return io_slice(self.cfg, kind, p, self.seed)
        if kind in NORM_KINDS:
            if self.banks is not None and (layer, sub, kind) in self.banks:
                b = self.banks[(layer, sub, kind)]
                return bf16_bits_to_f32(b) if b.dtype == np.uint16 else b
            return weight_slice(self.cfg, layer, sub, kind, p, self.seed)
        if self.banks is not None and (layer, sub, kind) in self.banks:
            b = self.banks[(layer, sub, kind)][p]
            return bf16_bits_to_f32(b) if b.dtype == np.uint16 else b
        return weight_slice(self.cfg, layer, sub, kind, p, self.seed)

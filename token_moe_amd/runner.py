"""Glue between a workload description and a libtmx context: build the
tmx_config, upload the seeded weight banks. Marshalling only -- every step
of the forward runs in libtmx.so."""
from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np

from . import tmx

# weight kinds use the same numbering in the seeded generator and tmx.h


def config_from_workload(wl, B_max: Optional[int] = None) -> tmx.tmx_config:
    return tmx.make_config(
        B_max=B_max or wl.B, T=wl.T, H=wl.H, D=wl.D, L=wl.L,
        hidden_mix=wl.hidden_mix, hidden_rev=wl.hidden_rev, E=wl.E, top_k=wl.top_k,
        expert_hidden=wl.expert_hidden, shared_hidden=wl.shared_hidden, alpha=wl.alpha,
        eps=wl.eps, inter_residual_gap=wl.gap,
        dtype={"bf16": tmx.TMX_BF16, "mxfp8": tmx.TMX_MXFP8}.get(wl.dtype, tmx.TMX_F32),
        block=tmx.TMX_BLOCK_RANKMIXER if getattr(wl, "rankmixer", False) else tmx.TMX_BLOCK_TOKENMIXER_LARGE)


def torch_dtype(wl):
    import torch
    return torch.bfloat16 if wl.bf16_values else torch.float32


def host_tensor(wl, a: np.ndarray):
    """Numpy array -> contiguous CPU torch tensor of the workload dtype.
    uint16 arrays are taken as bf16 bit patterns; float arrays as values
    (already representable in the workload dtype)."""
    import torch
    if a.dtype == np.uint16:
        if not wl.bf16_values:
            raise ValueError("bf16 bit patterns given for a non-bf16 workload")
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch_dtype(wl)).contiguous()


def upload_weights(ctx: tmx.Context, wl, banks: Dict[Tuple[int, int, int], np.ndarray]):
    """banks: {(layer 1..L, sub, kind): fp32 array or CPU torch tensor}.
    Layer l of the pages is layer l-1 of the C ABI."""
    import torch
    for (layer, sub, kind), arr in banks.items():
        t = arr if isinstance(arr, torch.Tensor) else host_tensor(wl, arr)
        t = t.contiguous()
        ctx.load_weights(layer - 1, sub, kind, t.data_ptr(), t.numel() * t.element_size())


def make_context(wl, banks, B_max: Optional[int] = None, device: int = 0, io_banks=None) -> tmx.Context:
    """A context holding the workload's stack; with ``io_banks`` (a model
    workload's tokenizer and head banks, {(0, 0, kind): array}) also its
    front and back."""
    ctx = tmx.Context(config_from_workload(wl, B_max), device)
    upload_weights(ctx, wl, banks)
    if io_banks is not None:
        ctx.set_model_io(list(wl.groups), wl.tok_hidden, wl.head_hidden)
        for (_, _, kind), arr in io_banks.items():
            t = host_tensor(wl, arr).contiguous()
            ctx.load_io_weights(kind, t.data_ptr(), t.numel() * t.element_size())
    return ctx

"""Upload a drawn layer to device tensors in the library's storage formats.

Marshalling only: bf16 bit patterns become torch.bfloat16 tensors of the same
bits, fp16 bit patterns torch.float16, codes uint8, masks int64 (uint64 bits).
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import Layer, MoEConfig


def dims_dict(cfg: MoEConfig, **over) -> dict:
    d = dict(hidden=cfg.hidden, n_experts=cfg.n_experts, top_k=cfg.top_k, inter=cfg.inter,
             n_shared=cfg.n_shared, shared_inter=cfg.shared_inter, lore_rank=cfg.lore_rank,
             renormalize=cfg.renormalize, shared_gate=cfg.shared_gate, floe_keep=cfg.floe_keep,
             dtype=cfg.dtype, up_format=cfg.up_format)
    d.update(over)
    return d


def tensor(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Storage array -> device tensor holding the same bits."""
    a = np.ascontiguousarray(a)
    if dtype == "bf16" and a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.uint16:           # fp16 bit patterns
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.float16)
    return torch.from_numpy(a).to(device)


def mask_tensor(masks, device) -> torch.Tensor:
    """uint64 bit masks (Python ints) -> int64 device tensor with the same bits."""
    arr = np.array([int(m) for m in np.atleast_1d(masks)], dtype=np.uint64).view(np.int64)
    return torch.from_numpy(arr).to(device)


def upload(layer: Layer, device="cuda", names=None) -> Dict[str, torch.Tensor]:
    cfg = layer.cfg
    out = {"w_router": tensor(layer.w_router(), cfg.dtype, device)}
    if cfg.shared_gate:
        out["w_shared_gate"] = tensor(layer.w_shared_gate(), cfg.dtype, device)
    if cfg.prefetch:
        out["w_prefetch"] = tensor(layer.w_prefetch(), cfg.dtype, device)
    for n in (names or layer.tensor_names()):
        out[n] = tensor(layer.full(n), cfg.dtype, device)
    return out

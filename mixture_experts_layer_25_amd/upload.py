"""Copy synthetic host inputs (raw bits) to device tensors for libmoe."""
from __future__ import annotations

import numpy as np
import torch

from . import moe, synthetic as syn


def _dev_bits(a: np.ndarray, device) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.uint8:
        return torch.from_numpy(a).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def cfg_of(c: syn.Config) -> moe.Cfg:
    return moe.Cfg(c.T, c.D, c.E, c.F, c.k, c.gating, c.renorm, c.capacity, c.clamp, c.act,
                   c.wdt, c.shared_F)


def to_device(inp: syn.Inputs, device="cuda"):
    """Returns (cfg, x, W_r, bias, Weights) on `device`."""
    x = _dev_bits(inp.x, device)
    W_r = _dev_bits(inp.W_r, device)
    bias = _dev_bits(inp.bias, device) if inp.bias is not None else None
    w = moe.Weights(W_gate=_dev_bits(inp.W_gate, device), W_up=_dev_bits(inp.W_up, device),
                    W_down=_dev_bits(inp.W_down, device))
    if inp.S_gate is not None:
        w.S_gate = _dev_bits(inp.S_gate, device)
        w.S_up = _dev_bits(inp.S_up, device)
        w.S_down = _dev_bits(inp.S_down, device)
    if inp.Ws_gate is not None:
        w.Ws_gate = _dev_bits(inp.Ws_gate, device)
        w.Ws_up = _dev_bits(inp.Ws_up, device)
        w.Ws_down = _dev_bits(inp.Ws_down, device)
    return cfg_of(inp.cfg), x, W_r, bias, w


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy raw bits (bf16 -> uint16)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()

"""Move generated inputs to the device (plumbing shared by the GPU tests and the bench)."""

from __future__ import annotations

import torch

from .generate import Inputs


def to_device(inp: Inputs, device="cuda") -> dict:
    """Device copies of every input, laid out as the C ABI expects."""
    wl = inp.wl
    d = {
        "xq": inp.xq.to(device, non_blocking=False).contiguous(),
        "xp": inp.xp.to(device).contiguous(),
        "W": inp.W.to(device).contiguous(),
        "targets": inp.targets.to(device).contiguous(),
        "mask": inp.mask.to(device).contiguous(),
        "rewards": inp.rewards.to(device).contiguous(),
        "S": wl.S, "L": wl.L, "H": wl.H, "V": wl.V,
    }
    return d

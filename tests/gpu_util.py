"""Helpers for the GPU tests: seeded inputs as device tensors, error metrics."""

from __future__ import annotations

import sys

import numpy as np

import seeded_inputs as si


def announce(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a lost box still says where it was."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def dev_tensor(arrays: dict, name: str, dtype: str):
    """Device tensor of a seeded array (bf16 from its exact bits, or float32)."""
    torch = torch_mod()
    if dtype == "bf16":
        bits = np.ascontiguousarray(arrays[name + "_bits"])
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arrays[name], dtype=np.float32)).cuda()


def bf16_from_f32(x: np.ndarray):
    torch = torch_mod()
    bits, vals = si.bf16_round(np.asarray(x, dtype=np.float32))
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda(), vals


def host(t) -> np.ndarray:
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def max_abs(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.max(np.where(np.isnan(d), np.inf, d)))


def bf16_ulp(x) -> np.ndarray:
    """Spacing of bf16 values at |x| (8 significant bits)."""
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)

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


def grad_rounding_bound(q, k, v, o, lse, do, scale: float, causal: bool):
    """Per-element bound on the bf16 backward's own rounding, for one head.

    The kernel rounds P and dS to bf16 (relative error <= 2^-9 each) before
    the products dV = P^T dO, dK = scale dS^T Q and dQ = scale dS K, which
    accumulate in float32. Rounding an operand moves a sum of products by at
    most 2^-9 times the sum of their absolute values, so with a 2x margin:
      |d(dQ)| <= 2^-8 scale (|dS| |K|),  |d(dK)| <= 2^-8 scale (|dS|^T |Q|),
      |d(dV)| <= 2^-8 (|P|^T |dO|).
    With cancellation in dS K these exceed one bf16 spacing of the result.
    Returns (bq, bk, bv) shaped like dQ, dK, dV.
    """
    q, k, v, o, do = (np.asarray(a, np.float64) for a in (q, k, v, o, do))
    n = q.shape[0]
    s = scale * (q @ k.T)
    if causal:
        s = np.where(np.tril(np.ones((n, n), bool)), s, -np.inf)
    p = np.exp(s - np.asarray(lse, np.float64)[:, None])
    ds = np.abs(p * (do @ v.T - np.sum(do * o, axis=1)[:, None]))
    u = 2.0 ** -8
    return u * scale * (ds @ np.abs(k)), u * scale * (ds.T @ np.abs(q)), u * (np.abs(p).T @ np.abs(do))

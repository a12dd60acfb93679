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


def saved_inputs_bound(q, k, v, do, scale: float, causal: bool, tol_o: float, tol_l: float):
    """Per-element bound on the backward from a forward's saved O and L, for one head.

    All inputs are the oracle's: q, k, v, do as the GPU sees them, O and L
    recomputed here from the plain definition. The backward takes the saved O
    and L of a forward whose O is within tol_o and whose L is within tol_l of
    the exact values (each asserted by the caller before this bound is used).
    With the exact P, dS and D of the oracle:
      * an error |dL| <= tol_l in L changes P = exp(S - L) by a factor
        exp(-dL), so |P' - P| <= r P with r = expm1(tol_l);
      * an error of at most tol_o in each element of O moves
        D_i = rowsum(dO_i * O_i) by at most dD_i = tol_o * sum_k |dO_ik|;
      * dS' - dS = P rho (dP - D) - P (1 + rho) dD, so
        |dS' - dS| <= E = r |dS| + (1 + r) P dD and |dS'| <= |dS| + E;
      * dQ = scale dS K, dK = scale dS^T Q and dV = P^T dO are linear in dS
        and P, so the propagated error is scale E |K|, scale E^T |Q| and
        r P^T |dO|;
      * the kernel's own bf16 rounding of P' and dS' adds the bound of
        grad_rounding_bound taken on |P'| <= (1 + r) P and |dS'| <= |dS| + E.
    Returns (bq, bk, bv) shaped like dQ, dK, dV.
    """
    q, k, v, do = (np.asarray(a, np.float64) for a in (q, k, v, do))
    n = q.shape[0]
    s = scale * (q @ k.T)
    if causal:
        s = np.where(np.tril(np.ones((n, n), bool)), s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / np.sum(e, axis=1, keepdims=True)
    o = p @ v
    ds = np.abs(p * (do @ v.T - np.sum(do * o, axis=1)[:, None]))
    r = float(np.expm1(tol_l))
    dd = tol_o * np.sum(np.abs(do), axis=1)
    err = r * ds + (1.0 + r) * p * dd[:, None]
    ds_max = ds + err
    p_max = (1.0 + r) * p
    u = 2.0 ** -8
    ak, aq, ado = np.abs(k), np.abs(q), np.abs(do)
    bq = scale * (err @ ak) + u * scale * (ds_max @ ak)
    bk = scale * (err.T @ aq) + u * scale * (ds_max.T @ aq)
    bv = r * (p.T @ ado) + u * (p_max.T @ ado)
    return bq, bk, bv

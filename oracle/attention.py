"""Plain float64 definition of exact attention, forward and backward.

TEST INFRASTRUCTURE. Nothing on the product path may import this module:
only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it. It shares no code with the HIP library.

Everything here is the plain definition written out in numpy float64 on the
CPU: the full score row, the three-pass safe softmax, the product with V and
the log-sum-exp. No tiling, no online recurrence and no reordering beyond
splitting the query rows into independent chunks to bound memory (each chunk
holds whole rows, so the chunking does not change what a row computes).

Sources (the pages this follows):
  * "FlashAttention v1～v4 完整进化史", section "第一层地基：注意力到底在算什么":
    S = Q K^T / sqrt(d), P = softmax(S), O = P V, Q/K/V of shape N x d.
  * "6.1 FlashAttention V1详解", section 8.1: tensors are [B, H, N, D], batch
    and head pass through as batch dimensions.
  * "6.1 FlashAttention V1详解", section 3.1: safe softmax in three passes
    (row max, exponent sum, normalise).
  * "FlashAttention v1～v4 完整进化史", v2 part 1: one statistic per row is
    kept, the log-sum-exp L = m + log(l).
  * "6.1 FlashAttention V1详解", section 6.1: dV = P^T dO, dP = dO V^T,
    dS = P * (dP - rowsum(dO * O)); the identity rowsum(dP*P) = rowsum(dO*O).
    dQ = scale * dS K and dK = scale * dS^T Q follow from S = scale * Q K^T by
    the chain rule (the pages name five matrix products for the backward in
    "FlashAttention v1～v4 完整进化史", v4 part 4, and print only three).

Readings where the pages are silent:
  * causal mask: key j is visible to query i when j <= i (diagonal kept);
  * a row with no visible key has O = 0 and LSE = -inf (not reachable when
    the number of queries equals the number of keys, since key 0 is visible);
  * scale is an explicit argument (the workloads use 1/sqrt(d)).

Pins: tests/test_oracle_pins.py (worked example, closed forms, brute force,
finite differences, CPU library routine, invariances).
"""

from __future__ import annotations

import numpy as np

__all__ = ["scores", "safe_softmax", "forward", "backward", "forward_rows",
           "backward_head", "kv_head", "forward_gqa", "backward_gqa", "forward_varlen",
           "backward_varlen"]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def scores(q_rows: np.ndarray, k: np.ndarray, scale: float, causal: bool,
           row0: int = 0) -> np.ndarray:
    """S = scale * Q K^T for query rows row0 .. row0+len(q_rows)-1 of one head.

    With ``causal`` the entries with key index j > query index i are -inf.
    """
    s = float(scale) * (_f64(q_rows) @ _f64(k).T)
    if causal:
        i = np.arange(row0, row0 + s.shape[0])[:, None]
        j = np.arange(s.shape[1])[None, :]
        s = np.where(j > i, -np.inf, s)
    return s


def safe_softmax(s: np.ndarray):
    """Row-wise safe softmax in three passes.

    Pass 1: m = max_j s_j. Pass 2: l = sum_j exp(s_j - m). Pass 3: p = exp(s - m) / l.
    Returns (p, m, l). Rows with m = -inf (nothing visible) give p = 0, l = 0.
    """
    m = s.max(axis=1)
    finite = np.isfinite(m)
    m_use = np.where(finite, m, 0.0)
    e = np.exp(s - m_use[:, None])          # exp(-inf) = 0 for masked entries
    l = e.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(finite[:, None], e / np.where(finite, l, 1.0)[:, None], 0.0)
    return p, m, l


def _head_forward(q, k, v, scale, causal, row_chunk):
    n = q.shape[0]
    o = np.zeros((n, v.shape[1]), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        s = scores(q[r0:r1], k, scale, causal, r0)
        p, m, l = safe_softmax(s)
        o[r0:r1] = p @ v
        with np.errstate(divide="ignore"):
            lse[r0:r1] = np.where(np.isfinite(m), m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def forward(q, k, v, scale: float, causal: bool = False, row_chunk: int = 1024):
    """Exact attention for [B, H, N, d] (or [N, d]) inputs.

    Returns (O, LSE) in float64: O has the shape of q, LSE drops the last axis.
    LSE is the natural log of sum_j exp(S_ij) over the visible keys.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim == 2:
        o, lse = _head_forward(q, k, v, scale, causal, row_chunk)
        return o, lse
    B, H, N, _ = q.shape
    o = np.empty(q.shape[:-1] + (v.shape[-1],), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = _head_forward(q[b, h], k[b, h], v[b, h], scale, causal, row_chunk)
    return o, lse


def forward_rows(q_head, k_head, v_head, rows, scale: float, causal: bool):
    """O and LSE of selected query rows of one head (for sampled checks).

    ``rows`` is a 1-D integer array of query indices; every row is computed
    from its full score row, independently of the others.
    """
    q_head, k_head, v_head = _f64(q_head), _f64(k_head), _f64(v_head)
    rows = np.asarray(rows, dtype=np.int64)
    s = float(scale) * (q_head[rows] @ k_head.T)
    if causal:
        j = np.arange(k_head.shape[0])[None, :]
        s = np.where(j > rows[:, None], -np.inf, s)
    p, m, l = safe_softmax(s)
    with np.errstate(divide="ignore"):
        lse = np.where(np.isfinite(m), m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return p @ v_head, lse


def backward_head(q, k, v, do, scale: float, causal: bool, row_chunk: int = 1024):
    """Gradients (dQ, dK, dV) of sum(O * dO) for one head, float64.

    P is recomputed from the full score rows; D_i = rowsum(dO_i * O_i) with the
    exact O. Row chunks accumulate dK and dV in float64.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    n = q.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        s = scores(q[r0:r1], k, scale, causal, r0)
        p, _, _ = safe_softmax(s)
        o = p @ v
        d_rows = np.sum(do[r0:r1] * o, axis=1)            # D_i = rowsum(dO * O)
        dv += p.T @ do[r0:r1]                              # dV = P^T dO
        dp = do[r0:r1] @ v.T                               # dP = dO V^T
        ds = p * (dp - d_rows[:, None])                    # dS = P * (dP - D)
        dq[r0:r1] = float(scale) * (ds @ k)                # dQ = scale dS K
        dk += float(scale) * (ds.T @ q[r0:r1])             # dK = scale dS^T Q
    return dq, dk, dv


def backward_from_saved(q, k, v, o, lse, do, scale: float, causal: bool = False):
    """Gradients of one head (or [B, H, N, d] inputs) from the saved O and L.

    The backward pass as the pages state it ("6.1 FlashAttention V1详解",
    sections 6.1-6.2): it takes Q, K, V, dO and the forward's saved O and
    statistics, recomputes P = exp(S - L) from the scores and L, and forms
    D = rowsum(dO * O) from the given O. With the exact O and L this equals
    ``backward``; given a rounded O (a bf16 forward's output) it is the exact
    result of the backward step on that input.
    """
    q, k, v, o, do = _f64(q), _f64(k), _f64(v), _f64(o), _f64(do)
    lse = _f64(lse)
    if q.ndim == 4:
        out = [np.empty_like(q), np.empty_like(k), np.empty_like(v)]
        for b in range(q.shape[0]):
            for h in range(q.shape[1]):
                g = backward_from_saved(q[b, h], k[b, h], v[b, h], o[b, h], lse[b, h], do[b, h], scale, causal)
                for t, x in zip(out, g):
                    t[b, h] = x
        return tuple(out)
    s = scores(q, k, scale, causal, 0)
    with np.errstate(invalid="ignore"):
        p = np.where(np.isfinite(s), np.exp(s - lse[:, None]), 0.0)   # P = exp(S - L)
    d_rows = np.sum(do * o, axis=1)                                    # D = rowsum(dO * O)
    dv = p.T @ do                                                      # dV = P^T dO
    dp = do @ v.T                                                      # dP = dO V^T
    ds = p * (dp - d_rows[:, None])                                    # dS = P * (dP - D)
    return float(scale) * (ds @ k), float(scale) * (ds.T @ q), dv      # dQ, dK, dV


def backward(q, k, v, do, scale: float, causal: bool = False, row_chunk: int = 1024):
    """Gradients for [B, H, N, d] (or [N, d]) inputs; see ``backward_head``."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    if q.ndim == 2:
        return backward_head(q, k, v, do, scale, causal, row_chunk)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    B, H = q.shape[:2]
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = backward_head(
                q[b, h], k[b, h], v[b, h], do[b, h], scale, causal, row_chunk)
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Grouped-query (GQA) and multi-query (MQA) attention.
#
# "FlashAttention v1～v4 完整进化史" names MQA and GQA ("最容易误解的六件事",
# third item; and the closing list of features to check a backend for) without
# defining them. Reading: the H query heads are split into H_kv groups of
# G = H / H_kv consecutive heads, and every head of group j attends with K and
# V head j (MQA: H_kv = 1; H_kv = H is ordinary multi-head attention). Each
# query head computes exactly the attention above with its group's K and V; a
# K or V head read by several query heads receives the sum of their gradients
# (the chain rule for a shared input).


def kv_head(h: int, H: int, H_kv: int) -> int:
    """K/V head read by query head h (groups of H / H_kv consecutive heads)."""
    if H_kv < 1 or H % H_kv:
        raise ValueError(f"H = {H} is not a multiple of H_kv = {H_kv}")
    return h // (H // H_kv)


def forward_gqa(q, k, v, scale: float, causal: bool = False, row_chunk: int = 1024):
    """(O, LSE) for q [B, H, N, d] with k, v [B, H_kv, N, d]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, _ = q.shape
    H_kv = k.shape[1]
    o = np.empty(q.shape[:-1] + (v.shape[-1],), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            j = kv_head(h, H, H_kv)
            o[b, h], lse[b, h] = _head_forward(q[b, h], k[b, j], v[b, j], scale, causal, row_chunk)
    return o, lse


def backward_gqa(q, k, v, do, scale: float, causal: bool = False, row_chunk: int = 1024):
    """(dQ, dK, dV): dQ per query head; dK, dV [B, H_kv, N, d] summed over the
    query heads of each group, in ascending head order."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H = q.shape[:2]
    H_kv = k.shape[1]
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            j = kv_head(h, H, H_kv)
            dq[b, h], dk_h, dv_h = backward_head(q[b, h], k[b, j], v[b, j], do[b, h], scale, causal, row_chunk)
            dk[b, j] += dk_h
            dv[b, j] += dv_h
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Variable-length batches packed along the sequence axis.
#
# "FlashAttention v1～v4 完整进化史" (v4 part 4) names variable-length
# sequences as a source of load imbalance, and its closing checklist lists
# them among backend features, without a layout. Reading: B sequences of
# lengths n_b are packed one after another, rows cu[b] .. cu[b+1]-1 of every
# head (cu = cumulative lengths, cu[0] = 0, cu[B] = T), q, o [H, T, d] and
# k, v [H_kv, T, d]; a query attends only to the keys of its own sequence
# (and, causal, to those at or before its own position in it). Heads map to
# K/V heads as in forward_gqa.


def forward_varlen(q, k, v, cu_seqlens, scale: float, causal: bool = False, row_chunk: int = 1024):
    """(O [H, T, d], LSE [H, T]) of packed sequences."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = [int(x) for x in cu_seqlens]
    H, T, _ = q.shape
    H_kv = k.shape[0]
    o = np.zeros(q.shape[:-1] + (v.shape[-1],), dtype=np.float64)
    lse = np.full((H, T), -np.inf, dtype=np.float64)
    for b in range(len(cu) - 1):
        r0, r1 = cu[b], cu[b + 1]
        if r1 <= r0:
            continue
        for h in range(H):
            j = kv_head(h, H, H_kv)
            o[h, r0:r1], lse[h, r0:r1] = _head_forward(q[h, r0:r1], k[j, r0:r1], v[j, r0:r1], scale, causal,
                                                       row_chunk)
    return o, lse


def backward_varlen(q, k, v, do, cu_seqlens, scale: float, causal: bool = False, row_chunk: int = 1024):
    """(dQ [H, T, d], dK, dV [H_kv, T, d]) of packed sequences; dK, dV of a
    shared K/V head sum its query heads in ascending order."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    cu = [int(x) for x in cu_seqlens]
    H = q.shape[0]
    H_kv = k.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(len(cu) - 1):
        r0, r1 = cu[b], cu[b + 1]
        if r1 <= r0:
            continue
        for h in range(H):
            j = kv_head(h, H, H_kv)
            g = backward_head(q[h, r0:r1], k[j, r0:r1], v[j, r0:r1], do[h, r0:r1], scale, causal, row_chunk)
            dq[h, r0:r1] = g[0]
            dk[j, r0:r1] += g[1]
            dv[j, r0:r1] += g[2]
    return dq, dk, dv

"""Pin checks for the float64 oracle.

Each check takes the function under test (the oracle's, or a copy with a
planted mistake) and raises AssertionError when the function disagrees with
something fixed independently of it: a value the pages print, a closed form,
brute force on tiny inputs, finite differences, or a CPU library routine.
tests/test_oracle_pins.py runs them on the oracle; tests/test_oracle_mutations.py
plants mistakes in copies of the oracle and requires that some check fails.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _expr(s: str) -> float:
    return float(eval(s, {"__builtins__": {}}, {"exp": math.exp}))


def worked_example():
    with open(os.path.join(GOLDEN, "online_softmax_worked_example.json")) as f:
        return json.load(f)


# ---------------------------------------------------------------- forward

def check_worked_example_forward(fwd):
    """A one-query problem whose scores are the page's [1, 2, 0, 3].

    q = [1], keys 1, 2, 0, 3 (d = 1, scale 1) and V = identity, so row 0 of O
    is the softmax itself and LSE = m + ln l.
    """
    g = worked_example()
    x = np.array(g["vector"])
    l_final = _expr(g["l_final_equals_expr"])
    m_final = g["m_after_block"][-1]
    q = np.array([[1.0]])
    k = x[:, None]
    v = np.eye(4)
    o, lse = fwd(q, k, v, 1.0, False)
    want_p = np.array([math.exp(xi - m_final) / l_final for xi in x])
    assert np.max(np.abs(o[0] - want_p)) <= 1e-15, (o, want_p)
    assert abs(lse[0] - (m_final + math.log(l_final))) <= 1e-14


def brute_force(q, k, v, scale, causal):
    """Pure-Python loops with the unshifted softmax exp(s) / sum exp(s)."""
    n, d = len(q), len(q[0])
    dv = len(v[0])
    o = [[0.0] * dv for _ in range(n)]
    lse = [0.0] * n
    for i in range(n):
        ws = []
        for j in range(len(k)):
            if causal and j > i:
                ws.append(0.0)
                continue
            s = scale * sum(q[i][t] * k[j][t] for t in range(d))
            ws.append(math.exp(s))
        z = sum(ws)
        lse[i] = math.log(z)
        for c in range(dv):
            o[i][c] = sum(ws[j] * v[j][c] for j in range(len(k))) / z
    return np.array(o), np.array(lse)


def check_brute_force(fwd):
    rng = _rng(11)
    for n, d, dv, causal, scale in [(1, 1, 1, False, 0.7), (3, 2, 3, False, 0.5),
                                    (5, 3, 2, True, 1.3), (4, 3, 4, True, 0.25),
                                    (5, 2, 2, False, 2.0)]:
        q = rng.standard_normal((n, d))
        k = rng.standard_normal((n, d))
        v = rng.standard_normal((n, dv))
        o, lse = fwd(q, k, v, scale, causal)
        ob, lb = brute_force(q.tolist(), k.tolist(), v.tolist(), scale, causal)
        assert np.max(np.abs(o - ob)) <= 1e-12, (n, d, causal)
        assert np.max(np.abs(lse - lb)) <= 1e-12, (n, d, causal)


def check_closed_forms(fwd):
    rng = _rng(12)
    # N = 1: O = V, LSE = scale q.k
    q, k, v = rng.standard_normal((3, 1, 8))
    o, lse = fwd(q, k, v, 0.3, False)
    assert np.max(np.abs(o - v)) <= 1e-15
    assert abs(lse[0] - 0.3 * float(q[0] @ k[0])) <= 1e-14
    # causal row 0 sees only key 0
    n, d = 9, 5
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    o, lse = fwd(q, k, v, 0.4, True)
    assert np.max(np.abs(o[0] - v[0])) <= 1e-15
    assert abs(lse[0] - 0.4 * float(q[0] @ k[0])) <= 1e-14
    # scale 0: uniform weights; mean of V (prefix means when causal); LSE = ln(#keys)
    o, lse = fwd(q, k, v, 0.0, False)
    assert np.max(np.abs(o - v.mean(axis=0)[None, :])) <= 1e-14
    assert np.max(np.abs(lse - math.log(n))) <= 1e-14
    o, lse = fwd(q, k, v, 0.0, True)
    pref = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    assert np.max(np.abs(o - pref)) <= 1e-14
    assert np.max(np.abs(lse - np.log(np.arange(1, n + 1)))) <= 1e-14
    # identical keys: uniform weights whatever the query; LSE = s + ln(#keys)
    k1 = np.repeat(rng.standard_normal((1, d)), n, axis=0)
    o, lse = fwd(q, k1, v, 0.5, False)
    assert np.max(np.abs(o - v.mean(axis=0)[None, :])) <= 1e-13
    assert np.max(np.abs(lse - (0.5 * (q @ k1[0]) + math.log(n)))) <= 1e-13


def check_torch_cpu(fwd):
    """Compare with torch's CPU scaled_dot_product_attention in float64."""
    import torch
    rng = _rng(13)
    for (B, H, N, d, causal, scale) in [(2, 3, 17, 8, False, 0.35), (1, 2, 33, 16, True, 0.25),
                                        (2, 1, 64, 4, True, 1.0)]:
        q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
        o, lse = fwd(q, k, v, scale, causal)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
        s = scale * (tq @ tk.transpose(-1, -2))
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
        tl = torch.logsumexp(s, dim=-1)
        assert np.max(np.abs(o - to.numpy())) <= 1e-12
        assert np.max(np.abs(lse - tl.numpy())) <= 1e-12


def check_invariances(fwd):
    rng = _rng(14)
    n, d = 24, 6
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    o, lse = fwd(q, k, v, 0.45, False)
    # key permutation (K and V rows together) leaves O and LSE unchanged
    perm = rng.permutation(n)
    o2, l2 = fwd(q, k[perm], v[perm], 0.45, False)
    assert np.max(np.abs(o - o2)) <= 1e-13 and np.max(np.abs(lse - l2)) <= 1e-13
    # query permutation permutes the rows of O
    o3, l3 = fwd(q[perm], k, v, 0.45, False)
    assert np.max(np.abs(o[perm] - o3)) <= 1e-13 and np.max(np.abs(lse[perm] - l3)) <= 1e-13
    # shifting every key by u shifts row i of S by scale q_i.u: O same, LSE + shift
    u = rng.standard_normal(d)
    o4, l4 = fwd(q, k + u[None, :], v, 0.45, False)
    assert np.max(np.abs(o - o4)) <= 1e-12
    assert np.max(np.abs(lse + 0.45 * (q @ u) - l4)) <= 1e-12
    # the same with shifts of up to +-2000 that differ from row to row: each row
    # must subtract its own maximum or its exponentials under- or overflow
    u = rng.standard_normal(d)
    u *= 2000.0 / (0.45 * np.max(np.abs(q @ u)))
    o4, l4 = fwd(q, k + u[None, :], v, 0.45, False)
    assert np.max(np.abs(o - o4)) <= 1e-9
    assert np.max(np.abs(lse + 0.45 * (q @ u) - l4)) <= 1e-9
    # orthogonal rotation of Q and K (incoherent processing identity)
    m, _ = np.linalg.qr(rng.standard_normal((d, d)))
    o5, l5 = fwd(q @ m, k @ m, v, 0.45, True)
    o6, l6 = fwd(q, k, v, 0.45, True)
    assert np.max(np.abs(o5 - o6)) <= 1e-10 and np.max(np.abs(l5 - l6)) <= 1e-10
    # O rows are convex combinations of V rows
    assert np.all(o <= v.max(axis=0) + 1e-12) and np.all(o >= v.min(axis=0) - 1e-12)


FORWARD_CHECKS = [check_worked_example_forward, check_brute_force, check_closed_forms,
                  check_torch_cpu, check_invariances]


# ---------------------------------------------------------------- backward

def _loss(fwd, q, k, v, do, scale, causal):
    o, _ = fwd(q, k, v, scale, causal)
    return float(np.sum(o * do))


def check_finite_differences(bwd, fwd):
    """Central differences of sum(O * dO), h = 1e-6, on tiny inputs."""
    rng = _rng(21)
    for n, d, causal, scale in [(5, 3, False, 0.6), (7, 4, True, 0.5), (8, 2, True, 1.1)]:
        q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
        dq, dk, dv = bwd(q, k, v, do, scale, causal)
        h = 1e-6
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp = x.copy(); xp[idx] += h
                xm = x.copy(); xm[idx] -= h
                args = {"q": q, "k": k, "v": v}
                args[name] = xp
                lp = _loss(fwd, args["q"], args["k"], args["v"], do, scale, causal)
                args[name] = xm
                lm = _loss(fwd, args["q"], args["k"], args["v"], do, scale, causal)
                fd[idx] = (lp - lm) / (2 * h)
            err = np.max(np.abs(fd - g)) / max(1.0, np.max(np.abs(fd)))
            assert err <= 1e-6, (name, n, d, causal, err)


def check_torch_autograd(bwd):
    import torch
    rng = _rng(22)
    for (N, d, causal, scale) in [(19, 8, False, 0.35), (40, 16, True, 0.25)]:
        q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
        dq, dk, dv = bwd(q, k, v, do, scale, causal)
        tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
        to = torch.nn.functional.scaled_dot_product_attention(
            tq[None, None], tk[None, None], tv[None, None], is_causal=causal, scale=scale)[0, 0]
        (to * torch.from_numpy(do)).sum().backward()
        for a, b in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            assert np.max(np.abs(a - b.numpy())) <= 1e-11


BACKWARD_CHECKS = [check_finite_differences, check_torch_autograd]

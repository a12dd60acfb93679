"""Pins of the oracle's packed variable-length attention.

The reading (each packed sequence attends only within itself, causal inside
it; heads map to K/V heads as in grouped-query attention) is checked against
PyTorch's CPU scaled_dot_product_attention over the whole packed axis with a
block-diagonal mask (values and autograd gradients), against central
differences, and against the plain oracle per sequence.
"""

import numpy as np
import pytest

from oracle import attention as A

LENS = [5, 1, 17, 0, 9]


def _inputs(rng, H, H_kv, T, d):
    return (rng.standard_normal((H, T, d)), rng.standard_normal((H_kv, T, d)), rng.standard_normal((H_kv, T, d)),
            rng.standard_normal((H, T, d)))


def _mask(cu, causal):
    T = cu[-1]
    seq = np.zeros(T, dtype=np.int64)
    for b in range(len(cu) - 1):
        seq[cu[b]:cu[b + 1]] = b
    m = seq[:, None] == seq[None, :]
    if causal:
        m &= np.arange(T)[None, :] <= np.arange(T)[:, None]
    return m


def check_sdpa(mod, H, H_kv, causal):
    import torch
    cu = np.concatenate([[0], np.cumsum(LENS)])
    T = int(cu[-1])
    rng = np.random.default_rng(51 + H + 3 * H_kv + causal)
    q, k, v, do = _inputs(rng, H, H_kv, T, 8)
    scale = 0.4
    o, lse = mod.forward_varlen(q, k, v, cu, scale, causal)
    dq, dk, dv = mod.backward_varlen(q, k, v, do, cu, scale, causal)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None], scale=scale,
                                                          attn_mask=torch.from_numpy(_mask(cu, causal)),
                                                          enable_gqa=True)[0]
    (to * torch.from_numpy(do)).sum().backward()
    assert np.max(np.abs(o - to.detach().numpy())) <= 1e-12
    for a, b in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(a - b.numpy())) <= 1e-11
    s = scale * np.einsum("htd,hsd->hts", q, np.repeat(k, H // H_kv, axis=0))
    s = np.where(_mask(cu, causal)[None], s, -np.inf)
    m = s.max(-1, keepdims=True)
    assert np.max(np.abs(lse - (m[..., 0] + np.log(np.exp(s - m).sum(-1))))) <= 1e-12


@pytest.mark.parametrize("H,H_kv,causal", [(2, 2, False), (2, 2, True), (4, 2, True), (3, 1, False)])
def test_varlen_matches_torch_sdpa_block_diagonal(H, H_kv, causal):
    check_sdpa(A, H, H_kv, causal)


def check_finite_differences(mod):
    rng = np.random.default_rng(61)
    cu = [0, 3, 4, 8]
    q, k, v, do = _inputs(rng, 2, 1, 8, 2)
    scale, causal, h = 0.8, True, 1e-6

    def loss(qq, kk, vv):
        o, _ = mod.forward_varlen(qq, kk, vv, cu, scale, causal)
        return float(np.sum(o * do))

    g = mod.backward_varlen(q, k, v, do, cu, scale, causal)
    for i, x in enumerate((q, k, v)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_p[i] = xp
            args_m = [q, k, v]
            args_m[i] = xm
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.max(np.abs(fd - g[i])) / max(1.0, np.max(np.abs(fd))) <= 1e-6, i


def test_varlen_finite_differences():
    check_finite_differences(A)


def test_varlen_is_per_sequence_attention():
    rng = np.random.default_rng(71)
    cu = [0, 4, 4, 11, 20]
    q, k, v, do = _inputs(rng, 2, 2, 20, 4)
    o, lse = A.forward_varlen(q, k, v, cu, 0.5, True)
    for b in range(4):
        r0, r1 = cu[b], cu[b + 1]
        if r1 == r0:
            continue
        o2, l2 = A.forward(q[None, :, r0:r1], k[None, :, r0:r1], v[None, :, r0:r1], 0.5, True)
        assert np.array_equal(o[:, r0:r1], o2[0]) and np.array_equal(lse[:, r0:r1], l2[0])


VARLEN_MUTANTS = {
    "sequences see each other": [("o[h, r0:r1], lse[h, r0:r1] = _head_forward(q[h, r0:r1], k[j, r0:r1], v[j, r0:r1]",
                                  "o[h, r0:r1], lse[h, r0:r1] = _head_forward(q[h, r0:r1], k[j, :r1], v[j, :r1]")],
    "dK of the last head only": [("dk[j, r0:r1] += g[1]", "dk[j, r0:r1] = g[1]")],
    "first sequence dropped": [("for b in range(len(cu) - 1):\n        r0, r1 = cu[b], cu[b + 1]\n        if r1 <= r0:\n            continue\n        for h in range(H):\n            j = kv_head(h, H, H_kv)\n            o[",
                                "for b in range(1, len(cu) - 1):\n        r0, r1 = cu[b], cu[b + 1]\n        if r1 <= r0:\n            continue\n        for h in range(H):\n            j = kv_head(h, H, H_kv)\n            o[")],
}


@pytest.mark.parametrize("name", sorted(VARLEN_MUTANTS))
def test_varlen_mutant_is_caught(name):
    import inspect
    import types
    src = inspect.getsource(A)
    for old, new in VARLEN_MUTANTS[name]:
        assert old in src, old
        src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle_attention_varlen_mutant")
    exec(compile(src, "oracle_attention_varlen_mutant", "exec"), mod.__dict__)
    failures = 0
    for check in [lambda: check_finite_differences(mod)] + [
            lambda c=c: check_sdpa(mod, *c) for c in [(2, 2, False), (4, 2, True)]]:
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            failures += 1
    assert failures > 0, name

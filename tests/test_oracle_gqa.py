"""Pins of the oracle's grouped-query (GQA) and multi-query (MQA) attention.

The reading (query head h uses K/V head h // (H / H_kv), groups of consecutive
heads; shared K/V heads receive the sum of their heads' gradients) is checked
against PyTorch's CPU scaled_dot_product_attention with enable_gqa, against
central differences, and against the plain multi-head oracle with the K/V
heads repeated.
"""

import numpy as np
import pytest

from oracle import attention as A

CASES = [(4, 2, False), (6, 3, True), (4, 1, True), (3, 3, False), (8, 2, True)]


def _inputs(rng, B, H, H_kv, N, d):
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H_kv, N, d))
    v = rng.standard_normal((B, H_kv, N, d))
    do = rng.standard_normal((B, H, N, d))
    return q, k, v, do


def check_sdpa(mod, H, H_kv, causal):
    import torch
    rng = np.random.default_rng(31 + H + 7 * H_kv)
    q, k, v, do = _inputs(rng, 2, H, H_kv, 23, 8)
    scale = 0.3
    o, lse = mod.forward_gqa(q, k, v, scale, causal)
    dq, dk, dv = mod.backward_gqa(q, k, v, do, scale, causal)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale,
                                                          enable_gqa=True)
    (to * torch.from_numpy(do)).sum().backward()
    assert np.max(np.abs(o - to.detach().numpy())) <= 1e-12
    for a, b in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(a - b.numpy())) <= 1e-11
    # LSE: the natural log of the visible exponentials of each row
    s = scale * np.einsum("bhnd,bhmd->bhnm", q, np.repeat(k, H // H_kv, axis=1))
    if causal:
        s = np.where(np.triu(np.ones((23, 23), bool), 1), -np.inf, s)
    m = s.max(-1, keepdims=True)
    assert np.max(np.abs(lse - (m[..., 0] + np.log(np.exp(s - m).sum(-1))))) <= 1e-12


@pytest.mark.parametrize("H,H_kv,causal", CASES)
def test_gqa_matches_torch_sdpa(H, H_kv, causal):
    check_sdpa(A, H, H_kv, causal)


def check_finite_differences(mod):
    """dK and dV of a K/V head shared by three query heads, by central differences."""
    rng = np.random.default_rng(41)
    q, k, v, do = _inputs(rng, 1, 6, 2, 5, 3)
    scale, causal, h = 0.7, True, 1e-6

    def loss(kk, vv):
        o, _ = mod.forward_gqa(q, kk, vv, scale, causal)
        return float(np.sum(o * do))

    _, dk, dv = mod.backward_gqa(q, k, v, do, scale, causal)
    for name, x, g in (("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            lp = loss(xp, v) if name == "k" else loss(k, xp)
            lm = loss(xm, v) if name == "k" else loss(k, xm)
            fd[idx] = (lp - lm) / (2 * h)
        assert np.max(np.abs(fd - g)) / max(1.0, np.max(np.abs(fd))) <= 1e-6, name


def test_gqa_finite_differences_on_shared_heads():
    check_finite_differences(A)


def test_gqa_equals_mha_with_repeated_heads():
    rng = np.random.default_rng(43)
    q, k, v, do = _inputs(rng, 2, 6, 2, 17, 4)
    G = 3
    o, lse = A.forward_gqa(q, k, v, 0.5, True)
    o2, lse2 = A.forward(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), 0.5, True)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    dq, dk, dv = A.backward_gqa(q, k, v, do, 0.5, True)
    dq2, dk2, dv2 = A.backward(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), do, 0.5, True)
    assert np.array_equal(dq, dq2)
    assert np.allclose(dk, dk2.reshape(2, 2, G, 17, 4).sum(2), rtol=0, atol=1e-13)
    assert np.allclose(dv, dv2.reshape(2, 2, G, 17, 4).sum(2), rtol=0, atol=1e-13)


def test_kv_head_mapping():
    assert [A.kv_head(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [A.kv_head(h, 4, 1) for h in range(4)] == [0, 0, 0, 0]
    assert [A.kv_head(h, 3, 3) for h in range(3)] == [0, 1, 2]
    with pytest.raises(ValueError):
        A.kv_head(0, 6, 4)


# Plausible mistakes planted in copies of the oracle: some pin above must fail.
GQA_MUTANTS = {
    "interleaved groups": [("return h // (H // H_kv)", "return h % H_kv")],
    "dK of the last head only": [("dk[b, j] += dk_h", "dk[b, j] = dk_h")],
    "dV of the first head only": [("dv[b, j] += dv_h", "dv[b, j] += dv_h if h % (H // H_kv) == 0 else 0")],
    "V head clipped to the query head": [("_head_forward(q[b, h], k[b, j], v[b, j]",
                                          "_head_forward(q[b, h], k[b, j], v[b, min(h, H_kv - 1)]")],
}


@pytest.mark.parametrize("name", sorted(GQA_MUTANTS))
def test_gqa_mutant_is_caught(name):
    import inspect
    import types
    src = inspect.getsource(A)
    for old, new in GQA_MUTANTS[name]:
        assert old in src, old
        src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle_attention_gqa_mutant")
    exec(compile(src, "oracle_attention_gqa_mutant", "exec"), mod.__dict__)
    failures = 0
    for check in [lambda: check_finite_differences(mod)] + [lambda c=c: check_sdpa(mod, *c) for c in CASES]:
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            failures += 1
    assert failures > 0, name

"""Pins of the error bounds the GPU gradient tests use (CPU only).

tests/gpu_util.py turns the stated forward tolerances and the kernel's bf16
rounding into per-element bounds on the gradients. Each bound is checked here
against an emulation of the error it claims to cover, built on the oracle's
backward step ("6.1 FlashAttention V1详解", sections 6.1-6.2):
  * grad_rounding_bound: P and dS rounded to bf16 before the three products;
  * saved_inputs_bound: O moved by the full O tolerance in the direction that
    moves D the most, and L moved by the full LSE tolerance.
Each bound must hold, must not be vacuous (the emulated error reaches a fair
fraction of it), and must fail when the term it adds is dropped.
"""

import math

import numpy as np
import pytest

import seeded_inputs as si
from gpu_util import grad_rounding_bound, saved_inputs_bound
from oracle import attention as A


def _bf16(x):
    return si.bf16_round(np.asarray(x, np.float64).astype(np.float32))[1].astype(np.float64)


def _probs(q, k, lse, scale, causal):
    n = q.shape[0]
    s = scale * (q @ k.T)
    if causal:
        s = np.where(np.tril(np.ones((n, n), bool)), s, -np.inf)
    return np.exp(s - lse[:, None])


def _inputs(seed, n=48, d=16, key_growth=0.0):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    k *= (1.0 + key_growth * np.arange(n) / n)[:, None]
    return q, k, v, do


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("growth", [0.0, 5.0])
def test_rounding_bound_covers_bf16_p_and_ds(causal, growth):
    q, k, v, do = _inputs(11 + int(growth), key_growth=growth)
    scale = 1.0 / math.sqrt(q.shape[1])
    o, lse = A.forward(q, k, v, scale, causal)
    p = _probs(q, k, lse, scale, causal)
    ds = p * (do @ v.T - np.sum(do * o, axis=1)[:, None])
    exact = (scale * ds @ k, scale * ds.T @ q, p.T @ do)
    pr, dsr = _bf16(p), _bf16(ds)
    rounded = (scale * dsr @ k, scale * dsr.T @ q, pr.T @ do)
    bound = grad_rounding_bound(q, k, v, o, lse, do, scale, causal)
    for name, a, b, bd in zip(("dQ", "dK", "dV"), rounded, exact, bound):
        err = np.abs(a - b)
        assert np.all(err <= bd), name
        # not vacuous: the worst element uses a fair share of its bound
        assert np.max(err / bd) > 0.02, name


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("growth", [0.0, 5.0])
def test_saved_inputs_bound_covers_tolerances(causal, growth):
    q, k, v, do = _inputs(21 + int(growth), key_growth=growth)
    scale = 1.0 / math.sqrt(q.shape[1])
    tol_o, tol_l = 2e-2, 1e-3
    o, lse = A.forward(q, k, v, scale, causal)
    exact = A.backward(q, k, v, do, scale, causal)
    bound = saved_inputs_bound(q, k, v, do, scale, causal, tol_o, tol_l)
    no_pert = saved_inputs_bound(q, k, v, do, scale, causal, 0.0, 0.0)
    worst = [0.0, 0.0, 0.0]
    beyond_rounding = [False, False]
    for so in (1.0, -1.0):
        for sl in (1.0, -1.0):
            # every O element moved by the full tolerance, aligned with dO
            # (the largest change of D), and every L by the full tolerance
            o_p = o + so * tol_o * np.sign(do)
            l_p = lse + sl * tol_l
            p_p = _probs(q, k, l_p, scale, causal)
            ds_p = p_p * (do @ v.T - np.sum(do * o_p, axis=1)[:, None])
            # the kernel's rounding on top of the moved inputs
            dsr, pr = _bf16(ds_p), _bf16(p_p)
            got = (scale * dsr @ k, scale * dsr.T @ q, pr.T @ do)
            for i, (a, b, bd) in enumerate(zip(got, exact, bound)):
                err = np.abs(a - b)
                assert np.all(err <= bd), ("dQ", "dK", "dV")[i]
                worst[i] = max(worst[i], float(np.max(err / bd)))
            for i in range(2):
                beyond_rounding[i] |= bool(np.any(np.abs(got[i] - exact[i]) > no_pert[i]))
    assert min(worst) > 0.02, worst
    # dropping the tolerance terms leaves dQ and dK uncovered
    assert all(beyond_rounding)


def test_saved_inputs_bound_reduces_to_rounding_bound():
    """At zero tolerances the saved-input bound is the rounding bound."""
    q, k, v, do = _inputs(5)
    scale = 0.3
    o, lse = A.forward(q, k, v, scale, True)
    a = saved_inputs_bound(q, k, v, do, scale, True, 0.0, 0.0)
    b = grad_rounding_bound(q, k, v, o, lse, do, scale, True)
    for x, y in zip(a, b):
        assert np.allclose(x, y, rtol=1e-12, atol=1e-15)

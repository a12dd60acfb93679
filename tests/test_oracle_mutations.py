"""Plant mistakes in copies of the oracle; some pin must catch each one.

Each mutant is the oracle's own source with one plausible mistake put in (a
dropped term, a wrong sign or index, a transposed operand). The pins in
oracle_checks must reject every mutant; a mutant they accept means the pins
are too weak to vouch for the oracle.
"""

import inspect
import types

import numpy as np
import pytest

import oracle_checks as oc
from oracle import attention as A


def _mutant_module(replacements):
    src = inspect.getsource(A)
    for old, new in replacements:
        assert old in src, f"mutation site not found: {old!r}"
        src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle_attention_mutant")
    exec(compile(src, "oracle_attention_mutant", "exec"), mod.__dict__)
    return mod


FORWARD_MUTANTS = {
    "scale dropped": [("s = float(scale) * (_f64(q_rows) @ _f64(k).T)", "s = (_f64(q_rows) @ _f64(k).T)")],
    "scale squared": [("s = float(scale) * (_f64(q_rows) @ _f64(k).T)",
                       "s = float(scale) ** 2 * (_f64(q_rows) @ _f64(k).T)")],
    "diagonal masked": [("s = np.where(j > i, -np.inf, s)", "s = np.where(j >= i, -np.inf, s)")],
    "upper triangle kept": [("s = np.where(j > i, -np.inf, s)", "s = np.where(j < i, -np.inf, s)")],
    "row max from column": [("m = s.max(axis=1)", "m = s.max(axis=0).max() + 0 * s[:, 0]")],
    "sum over wrong axis": [("l = e.sum(axis=1)", "l = e.sum(axis=0).sum() + 0 * e[:, 0]")],
    "no normalisation": [("e / np.where(finite, l, 1.0)[:, None]", "e")],
    "lse without log": [("m + np.log(np.where(l > 0, l, 1.0))", "m + np.where(l > 0, l, 1.0)")],
    "lse without max": [("lse[r0:r1] = np.where(np.isfinite(m), m + np.log",
                         "lse[r0:r1] = np.where(np.isfinite(m), 0 * m + np.log")],
    "P transposed": [("o[r0:r1] = p @ v", "o[r0:r1] = (p.T @ v) if p.shape[0] == p.shape[1] else p @ v[::-1]")],
    "keys reversed": [("s = float(scale) * (_f64(q_rows) @ _f64(k).T)",
                       "s = float(scale) * (_f64(q_rows) @ _f64(k)[::-1].T)")],
    "exp sign flipped": [("e = np.exp(s - m_use[:, None])", "e = np.exp(-(s - m_use[:, None]))")],
}


BACKWARD_MUTANTS = {
    "D term dropped": [("ds = p * (dp - d_rows[:, None])", "ds = p * dp")],
    "D sign flipped": [("ds = p * (dp - d_rows[:, None])", "ds = p * (dp + d_rows[:, None])")],
    "dQ without scale": [("dq[r0:r1] = float(scale) * (ds @ k)", "dq[r0:r1] = (ds @ k)")],
    "dK from dS not transposed": [("dk += float(scale) * (ds.T @ q[r0:r1])",
                                   "dk += float(scale) * (ds @ q[r0:r1]) if ds.shape[0] == ds.shape[1] else 0")],
    "dV uses P not P^T": [("dv += p.T @ do[r0:r1]", "dv += p @ do[r0:r1] if p.shape[0] == p.shape[1] else 0")],
    "dP uses V not V^T": [("dp = do[r0:r1] @ v.T", "dp = do[r0:r1] @ v[::-1].T")],
    "D from dO only": [("d_rows = np.sum(do[r0:r1] * o, axis=1)", "d_rows = np.sum(do[r0:r1], axis=1)")],
    "dK uses K": [("dk += float(scale) * (ds.T @ q[r0:r1])", "dk += float(scale) * (ds.T @ k[r0:r1])")],
}


def _fails_some_check(checks, *args):
    failures = 0
    for check in checks:
        try:
            check(*args)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failures += 1
    return failures


@pytest.mark.parametrize("name", sorted(FORWARD_MUTANTS))
def test_forward_mutant_is_caught(name):
    mod = _mutant_module(FORWARD_MUTANTS[name])

    def fwd(q, k, v, scale, causal):
        return mod.forward(q, k, v, scale, causal)

    with np.errstate(all="ignore"):
        assert _fails_some_check([lambda f=c: f(fwd) for c in oc.FORWARD_CHECKS]) > 0, name


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTANTS))
def test_backward_mutant_is_caught(name):
    mod = _mutant_module(BACKWARD_MUTANTS[name])

    def bwd(q, k, v, do, scale, causal):
        return mod.backward(q, k, v, do, scale, causal)

    def fwd(q, k, v, scale, causal):
        return A.forward(q, k, v, scale, causal)

    checks = [lambda: oc.check_finite_differences(bwd, fwd), lambda: oc.check_torch_autograd(bwd)]
    with np.errstate(all="ignore"):
        assert _fails_some_check(checks) > 0, name

"""Pins of the float64 oracle against what the pages and the mathematics fix."""

import math

import numpy as np
import pytest

import oracle_checks as oc
from oracle import attention as A
from oracle import online as T


def fwd(q, k, v, scale, causal):
    return A.forward(q, k, v, scale, causal)


def bwd(q, k, v, do, scale, causal):
    return A.backward(q, k, v, do, scale, causal)


@pytest.mark.parametrize("check", oc.FORWARD_CHECKS, ids=lambda c: c.__name__)
def test_forward_pins(check):
    check(fwd)


def test_backward_finite_differences():
    oc.check_finite_differences(bwd, fwd)


def test_backward_torch_autograd():
    oc.check_torch_autograd(bwd)


def test_worked_example_recurrence():
    """The page's blocks [1, 2] then [0, 3] ("FlashAttention v1～v4 完整进化史", v1 part 2)."""
    g = oc.worked_example()
    steps = T.online_softmax_blocks(g["vector"], g["blocks"])
    for (m, l), m_want, l_expr in zip(steps, g["m_after_block"], g["l_after_block_expr"]):
        assert m == m_want
        assert abs(l - oc._expr(l_expr)) <= 1e-15
    assert abs(steps[-1][1] - oc._expr(g["l_final_equals_expr"])) <= 1e-15
    # the final sum is the shifted exponent sum of the whole vector
    direct = sum(math.exp(x - 3.0) for x in g["vector"])
    assert abs(steps[-1][1] - direct) <= 1e-15


def test_per_element_recurrence_matches_blocks():
    """Block size 1 ("A · Flash Attention" section 2.2) equals any blocking."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal(37) * 4
    one = T.online_softmax_blocks(x, [1] * 37)[-1]
    blk = T.online_softmax_blocks(x, [5, 9, 1, 22])[-1]
    m = x.max()
    assert one[0] == m and blk[0] == m
    assert abs(one[1] - np.exp(x - m).sum()) <= 1e-13
    assert abs(blk[1] - np.exp(x - m).sum()) <= 1e-13


def test_softmax_rows_sum_to_one_and_shift_invariance():
    rng = np.random.default_rng(4)
    s = rng.standard_normal((16, 40)) * 10
    p, m, l = A.safe_softmax(s)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-12
    p2, _, _ = A.safe_softmax(s + rng.standard_normal((16, 1)) * 100)
    assert np.max(np.abs(p - p2)) <= 1e-12
    # large scores do not overflow: the maximum is subtracted first
    p3, _, _ = A.safe_softmax(s + 1000.0)
    assert np.all(np.isfinite(p3))


def test_fully_masked_row_reading():
    """A row with no visible key: O = 0, LSE = -inf (reading; the pages are silent)."""
    s = np.array([[-np.inf, -np.inf], [0.0, 1.0]])
    p, m, l = A.safe_softmax(s)
    assert np.all(p[0] == 0) and m[0] == -np.inf and l[0] == 0
    assert abs(p[1].sum() - 1.0) <= 1e-15


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("normalise", [False, True])
def test_tiled_equals_plain_for_all_tiles_and_orders(causal, normalise):
    """Tiling is exact: every (B_r, B_c) and key-tile order reaches the plain result."""
    rng = np.random.default_rng(5)
    n, d = 45, 7
    q, k, v = (rng.standard_normal((n, d)) * 2 for _ in range(3))
    o_ref, l_ref = A.forward(q, k, v, 0.6, causal)
    for br, bc in [(1, 1), (3, 5), (16, 16), (45, 45), (64, 7), (8, 64)]:
        t_c = -(-n // bc)
        for order in (None, list(range(t_c))[::-1], list(rng.permutation(t_c))):
            o, lse = T.tiled_forward(q, k, v, 0.6, causal, br, bc, kv_order=order,
                                     normalise_each_step=normalise)
            assert np.max(np.abs(o - o_ref)) <= 1e-12, (br, bc, order)
            assert np.max(np.abs(lse - l_ref)) <= 1e-12, (br, bc, order)


def test_tiled_invariants_are_checked():
    """exp arguments <= 0 and rescale factors <= 1 hold at every step (asserted inside)."""
    rng = np.random.default_rng(6)
    q, k, v = (rng.standard_normal((20, 4)) * 5 for _ in range(3))
    T.tiled_forward(q, k, v, 1.0, True, 4, 3, check_invariants=True)


def test_d_identity():
    """rowsum(dP * P) = rowsum(dO * O) ("6.1 FlashAttention V1详解" section 6.1)."""
    rng = np.random.default_rng(7)
    n, d = 30, 6
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    for causal in (False, True):
        s = A.scores(q, k, 0.5, causal)
        p, _, _ = A.safe_softmax(s)
        o = p @ v
        dp = do @ v.T
        assert np.max(np.abs((dp * p).sum(axis=1) - (do * o).sum(axis=1))) <= 1e-12


def test_forward_rows_matches_forward():
    rng = np.random.default_rng(8)
    q, k, v = (rng.standard_normal((50, 8)) for _ in range(3))
    rows = np.array([0, 7, 31, 49])
    for causal in (False, True):
        o, lse = A.forward(q, k, v, 0.3, causal, row_chunk=16)
        o2, l2 = A.forward_rows(q, k, v, rows, 0.3, causal)
        assert np.max(np.abs(o[rows] - o2)) <= 1e-13
        assert np.max(np.abs(lse[rows] - l2)) <= 1e-13


def test_row_chunking_does_not_change_rows():
    rng = np.random.default_rng(9)
    q, k, v, do = (rng.standard_normal((1, 2, 70, 8)) for _ in range(4))
    o1, l1 = A.forward(q, k, v, 0.3, True, row_chunk=7)
    o2, l2 = A.forward(q, k, v, 0.3, True, row_chunk=1024)
    assert np.max(np.abs(o1 - o2)) <= 1e-14 and np.max(np.abs(l1 - l2)) <= 1e-14
    g1 = A.backward(q, k, v, do, 0.3, True, row_chunk=9)
    g2 = A.backward(q, k, v, do, 0.3, True, row_chunk=1024)
    for a, b in zip(g1, g2):
        assert np.max(np.abs(a - b)) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_backward_from_saved_pins(causal):
    """The backward from the saved O and L ("6.1 FlashAttention V1详解", 6.1-6.2).

    * with the exact forward's O and L it is the gradient of ``backward``
      (itself pinned by finite differences and autograd);
    * it is linear in O through D only: perturbing O by delta changes dQ by
      -scale diag(rowsum(dO * delta)) P K and dK by the transpose form, and
      leaves dV unchanged;
    * shifting every L by c scales P, hence every gradient, by exp(-c).
    """
    rng = np.random.default_rng(77)
    n, d, scale = 19, 8, 0.4
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    o, lse = A.forward(q, k, v, scale, causal)
    g_saved = A.backward_from_saved(q, k, v, o, lse, do, scale, causal)
    g_ref = A.backward(q, k, v, do, scale, causal)
    for a, b in zip(g_saved, g_ref):
        assert np.max(np.abs(a - b)) <= 1e-12
    delta = 1e-3 * rng.standard_normal((n, d))
    g_pert = A.backward_from_saved(q, k, v, o + delta, lse, do, scale, causal)
    s = q @ k.T * scale
    if causal:
        s = np.where(np.tril(np.ones((n, n), bool)), s, -np.inf)
    p = np.exp(s - lse[:, None])
    dd = np.sum(do * delta, axis=1)
    want_dq = g_saved[0] - scale * (dd[:, None] * p) @ k
    want_dk = g_saved[1] - scale * (dd[:, None] * p).T @ q
    assert np.max(np.abs(g_pert[0] - want_dq)) <= 1e-12
    assert np.max(np.abs(g_pert[1] - want_dk)) <= 1e-12
    assert np.max(np.abs(g_pert[2] - g_saved[2])) == 0.0
    g_shift = A.backward_from_saved(q, k, v, o, lse + 0.7, do, scale, causal)
    for a, b in zip(g_shift, g_saved):
        assert np.max(np.abs(a - math.exp(-0.7) * b)) <= 1e-12

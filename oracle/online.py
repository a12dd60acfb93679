"""Tiled attention with the online softmax, float64, for the oracle's self-tests.

TEST INFRASTRUCTURE (see oracle/attention.py). This module is not the oracle
the GPU is compared with; it exists to pin that the tiled recurrence the
kernels implement reaches the plain definition exactly (up to rounding), for
every tile size and every order of key tiles.

Sources:
  * "6.1 FlashAttention V1详解", section 3.2: the recurrence over blocks,
    m_j = max(m_{j-1}, max x^(j)), l_j = l_{j-1} e^{m_{j-1}-m_j} + sum e^{x-m_j},
    and the normalised output update; section 3.3: the rescale identity
    e^{x-m_new} = e^{x-m_old} e^{m_old-m_new} is exact.
  * "A · Flash Attention", section 2.2: the same recurrence one element at a
    time (block size 1).
  * "6.1 FlashAttention V1详解", section 5.1 steps 1-5 (normalised O after
    every block) and section 5.3 (every exponent argument is <= 0 and the
    rescale factor is <= 1).
  * "FlashAttention v1～v4 完整进化史", v1 part 2 and the v1 pseudocode
    (unnormalised O, one division by l at the end) and v2 part 1 (that form
    plus one saved L = m + log l per row).
  * "6.1 FlashAttention V1详解", section 8.2: initial m = -inf, l = 0, so the
    first rescale factor is exp(-inf) = 0.

Reading where the pages are silent: when a row has seen only masked keys
(m = -inf) the rescale factor exp(-inf - (-inf)) is taken as 0 and the block's
exponentials are 0.
"""

from __future__ import annotations

import numpy as np

__all__ = ["online_softmax_blocks", "tiled_forward"]


class InvariantError(AssertionError):
    pass


def online_softmax_blocks(x, block_sizes):
    """Run the blockwise (m, l) recurrence over a 1-D vector.

    ``block_sizes`` partitions x into consecutive blocks. Returns the list of
    (m, l) after each block.
    """
    x = np.asarray(x, dtype=np.float64)
    m, l = -np.inf, 0.0
    out = []
    pos = 0
    for bs in block_sizes:
        blk = x[pos:pos + bs]
        pos += bs
        m_new = max(m, float(blk.max())) if blk.size else m
        alpha = 0.0 if m_new == -np.inf else float(np.exp(m - m_new))
        add = 0.0 if m_new == -np.inf else float(np.exp(blk - m_new).sum())
        l = l * alpha + add
        m = m_new
        out.append((m, l))
    if pos != x.size:
        raise ValueError("block sizes must cover the vector")
    return out


def tiled_forward(q, k, v, scale: float, causal: bool, B_r: int, B_c: int,
                  kv_order=None, normalise_each_step: bool = False,
                  check_invariants: bool = True):
    """Tiled exact attention of one head with the online softmax.

    Outer loop over query tiles of B_r rows, inner loop over key/value tiles
    of B_c rows visited in ``kv_order`` (default ascending). Per query tile
    the state is (m, l, O) per row, initialised to (-inf, 0, 0).

    normalise_each_step=False: O is kept unnormalised and divided by l once at
    the end (v2 form). True: O is renormalised after every tile (v1 form,
    "6.1 FlashAttention V1详解" section 5.1 step 5).

    Returns (O, LSE) with LSE = m + ln l.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, n_k = q.shape[0], k.shape[0]
    t_c = -(-n_k // B_c)
    order = list(range(t_c)) if kv_order is None else list(kv_order)
    if sorted(order) != list(range(t_c)):
        raise ValueError("kv_order must be a permutation of the key tiles")
    o_all = np.zeros((n, v.shape[1]))
    lse_all = np.empty(n)
    for r0 in range(0, n, B_r):
        r1 = min(n, r0 + B_r)
        q_i = q[r0:r1]
        m = np.full(r1 - r0, -np.inf)
        l = np.zeros(r1 - r0)
        o = np.zeros((r1 - r0, v.shape[1]))
        for j in order:
            c0, c1 = j * B_c, min(n_k, (j + 1) * B_c)
            s = scale * (q_i @ k[c0:c1].T)                         # step 1
            if causal:
                ii = np.arange(r0, r1)[:, None]
                jj = np.arange(c0, c1)[None, :]
                s = np.where(jj > ii, -np.inf, s)
            m_tile = s.max(axis=1)                                 # step 2
            m_new = np.maximum(m, m_tile)                          # step 3
            live = np.isfinite(m_new)
            m_ref = np.where(live, m_new, 0.0)
            with np.errstate(invalid="ignore"):
                alpha = np.where(live, np.exp(m - m_ref), 0.0)     # step 4
                arg = s - m_ref[:, None]
            p = np.where(live[:, None], np.exp(arg), 0.0)
            if check_invariants:
                finite_args = arg[np.isfinite(arg) & live[:, None]]
                if finite_args.size and finite_args.max() > 0.0:
                    raise InvariantError("exponent argument above 0")
                if np.any(alpha > 1.0):
                    raise InvariantError("rescale factor above 1")
            l_new = alpha * l + p.sum(axis=1)
            if normalise_each_step:                                # step 5, v1 form
                with np.errstate(invalid="ignore", divide="ignore"):
                    inv = np.where(l_new > 0, 1.0 / np.where(l_new > 0, l_new, 1.0), 0.0)
                o = (alpha * l * inv)[:, None] * o + (inv[:, None] * p) @ v[c0:c1]
            else:                                                  # v2 form
                o = alpha[:, None] * o + p @ v[c0:c1]
            m, l = m_new, l_new
        if not normalise_each_step:
            with np.errstate(invalid="ignore", divide="ignore"):
                o = np.where((l > 0)[:, None], o / np.where(l > 0, l, 1.0)[:, None], 0.0)
        o_all[r0:r1] = o
        with np.errstate(divide="ignore"):
            lse_all[r0:r1] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o_all, lse_all

"""Per-element error bound for the fp8 attention kernel against the oracle's fp8 emulation.

The kernel and the emulation (oracle/fp8.py, fp8_attention_tiled) take the
same steps on the same codes; they differ only in how the scores are formed:
  * the fp8 matrix cores sum the products of one 32x32x64 step with a
    reduced precision: measured on MI355X over several input mixes, the error
    of a 64-term step stays below 3.1e-4 of its largest absolute product and
    below 2.1e-4 of the sum of its absolute products. A score takes two steps
    (d = 128), so the bound uses min(EPS_SUM * sum|p|, 2 * EPS_MAX * max|p|)
    with EPS_SUM = 2^-11 and EPS_MAX = 2^-10 (about 2.3x and 3x the
    measurements);
  * the float32 scaling, exp2 and max steps add a few float32 roundings.
From a score error |dS_ij| <= delta_ij the bound follows the emulation's own
steps:
  * the running maximum after each tile moves by at most delta_i = max_j
    delta_ij; with the power-of-two reference (the running maximum rounded
    up to a whole power of two, reference="pow2" in the emulation) the
    kernel may therefore round a maximum within delta_i of a power of two to
    the neighbouring one: P' of that tile's keys then moves by an exact
    factor of 2, which cancels against the factor 2 in the accumulator's
    scale except in e4m3's subnormal range and at its top code, so both
    references are taken as candidates there;
  * P' = 448 exp(S - m) therefore moves by a factor of at most
    exp(eta_i), eta_i = 2 delta_i;
  * its e4m3 code can be any code between those of P' exp(-eta_i) and
    P' exp(eta_i);
  * the row sum l moves by the same factor, plus float32 summation;
  * the P V product adds EPS_MMA of the sum of its absolute products;
  * the bf16 output adds half a bf16 spacing.
Everything here is float64 numpy. It uses the oracle's e4m3 codec and
dequantisation, and only the codes, scales and parameters the emulation
itself receives.
"""

from __future__ import annotations

import numpy as np

from oracle import fp8 as F

EPS_MMA = 2.0 ** -11     # relative to the sum of absolute products
EPS_MAX = 2.0 ** -10     # relative to the largest absolute product of one step
U32 = 2.0 ** -24
LN2 = float(np.log(2.0))


def _bf16_half_ulp(x):
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 8)


def bound_rows(q8, sq, k8, sk, v8, sv, scale, causal, rows, B_c=64, reference="pow2"):
    """Bounds for |O_gpu - O_emul| ([len(rows), d]) and |LSE_gpu - LSE_emul| ([len(rows)]).

    q8..sv are the codes and scales of one (batch, head): [N, d] and [ceil(N/64)].
    Also returns the emulation's O for the rows, rebuilt from the same
    quantities, as a cross-check of the bound's inputs.
    """
    N, d = q8.shape
    rows = np.asarray(rows)
    qd = F.dequantize(q8[None, None], sq[None, None])[0, 0][rows]
    kd = F.dequantize(k8[None, None], sk[None, None])[0, 0]
    vd = F.dequantize(v8[None, None], sv[None, None])[0, 0]
    s = scale * (qd @ kd.T)
    sabs = scale * (np.abs(qd) @ np.abs(kd).T)
    pmax = np.empty_like(sabs)
    for c0 in range(0, len(rows), 16):
        pmax[c0:c0 + 16] = scale * np.max(np.abs(qd[c0:c0 + 16, None, :] * kd[None, :, :]), axis=2)
    keys = np.arange(N)
    vis = np.ones_like(s, dtype=bool)
    if causal:
        vis = keys[None, :] <= rows[:, None]
    s = np.where(vis, s, -np.inf)
    # score error: matrix-core accumulation + float32 scaling / exp2 arguments
    s_fin = np.where(vis, s, 0.0)
    mma = np.minimum(EPS_MMA * sabs, 2 * EPS_MAX * pmax)
    delta = np.where(vis, mma + 8 * U32 * (np.abs(s_fin) + 1.0), 0.0)
    dmax = delta.max(axis=1)
    eta = 2.0 * dmax
    # running maximum after each tile of B_c keys
    t_c = -(-N // B_c)
    tile_of = keys // B_c
    tmax = np.stack([s[:, t * B_c:(t + 1) * B_c].max(axis=1) for t in range(t_c)], axis=1)
    m_run = np.maximum.accumulate(tmax, axis=1)
    alt = np.zeros_like(m_run)                      # the other candidate reference, in powers of two
    if reference == "pow2":
        with np.errstate(invalid="ignore"):
            u = m_run / LN2                         # the running maximum in log2 units
            r = np.ceil(u)
            win = 1.5 * dmax[:, None] / LN2 + 1e-6
            alt = np.where(u - (r - 1.0) <= win, -1.0, np.where(r - u <= win, 1.0, 0.0))
            m_run = np.where(np.isfinite(m_run), r * LN2, m_run)
    elif reference != "exact":
        raise ValueError(reference)
    m_fin = m_run[:, -1]
    m_at = m_run[:, tile_of]                        # reference in force for key j
    alt_at = alt[:, tile_of]
    with np.errstate(invalid="ignore", over="ignore"):
        p = np.where(vis, np.exp(s - m_at), 0.0)     # P~ of the emulation
        w = np.where(vis, np.exp(m_at - m_fin[:, None]), 0.0)
    l = (p * w).sum(axis=1)
    pq = F.e4m3_decode(F.e4m3_encode(p.astype(np.float32) * np.float32(448.0)))
    e = np.exp(eta)[:, None]
    lo = F.e4m3_decode(F.e4m3_encode(np.minimum(p * 448.0 / e, 448.0)))
    hi = F.e4m3_decode(F.e4m3_encode(np.minimum(p * 448.0 * e, 448.0)))
    # the neighbouring reference: P' times 2^-alt, its code times 2^alt
    f = np.exp2(-alt_at)
    lo = np.minimum(lo, F.e4m3_decode(F.e4m3_encode(np.minimum(p * f * 448.0 / e, 448.0))) / f)
    hi = np.maximum(hi, F.e4m3_decode(F.e4m3_encode(np.minimum(p * f * 448.0 * e, 448.0))) / f)
    # weights of V_j in O: pq/448 * w / l; GPU: within the code range, with
    # the rescale factors and l each off by at most exp(eta) (plus summation)
    lsum = np.exp(eta + N * U32 * 4)[:, None]
    a = pq / 448.0 * w / l[:, None]
    a_hi = hi / 448.0 * w * e * lsum / l[:, None]
    a_lo = lo / 448.0 * w / (e * lsum) / l[:, None]
    da = np.maximum(a_hi - a, a - a_lo)
    vabs = np.abs(vd)
    o_emul = a @ vd
    ob = da @ vabs + EPS_MMA * (a_hi @ vabs) * 2.0
    ob += _bf16_half_ulp(np.abs(o_emul) + ob) + 1e-7
    lse = m_fin + np.log(l)
    lb = 3.0 * dmax + 4 * N * U32 + 4 * U32 * np.abs(lse) + 1e-6
    return ob, lb, o_emul, lse

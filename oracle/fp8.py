"""FP8 (e4m3) codec, block quantisation and the fp8 attention emulation.

TEST INFRASTRUCTURE (see oracle/attention.py).

Sources:
  * "FlashAttention v1～v4 完整进化史", v3 part 3 (FP8): each block gets its
    own scale instead of one per tensor (block quantisation); Q and K are both
    multiplied by one random orthogonal matrix M, which leaves Q K^T unchanged
    because M M^T = I (incoherent processing); the first product's fp32
    accumulator is turned into the operand of the second fp8 product, i.e. P
    itself goes to fp8.
  * The e4m3 format is not printed on the pages. Reading: the OCP 8-bit
    "e4m3fn" format - 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent field 0 holds subnormals m/8 * 2^-6; the code with all
    exponent and mantissa bits set is NaN; there is no infinity; the largest
    finite magnitude is 448. Encoding rounds to nearest, ties to even, after
    saturating magnitudes above 448 to 448.
  * Block granularity is not stated. Reading: one scale per 64 consecutive
    rows (all d columns) of one (batch, head). Per-tensor baseline: one s
    for the whole tensor.
  * The form of a block's scale is not stated either. Reading: s = amax /
    448 (float32(amax) / 448 rounded to float32), which puts the block's
    largest magnitude on the largest code; s = 1 when the block is all zero,
    and a nonzero block whose amax / 448 underflows gets 2^-149 (the
    smallest positive float32). A second form (pow2=True) takes the
    smallest power of two at or above that value, kept at or above 2^-126:
    it is the form the fp8 matrix cores accept as a block scale (an 8-bit
    exponent), so the product with V can be scaled tile by tile inside the
    instruction without touching the accumulator. The GPU path quantises V
    in that form and Q, K in the plain one. Measured with this oracle
    (oracle/fp8_granularity.py, the 4 x 32 x 8192 x 128 workload, 8 heads,
    rotated Q and K): RMSE of O 0.2311 with every scale plain, 0.2309 with
    V's a power of two, 0.2534 with all three powers of two (a power of two
    costs Q and K the exact top code of every block).
  * Where a float decides a code (the division x / s), it is taken in
    float32, the precision the GPU quantiser uses (x / s is exact when s is
    a power of two).
  * The reference P~ is taken against before its e4m3 rounding. The pages
    round P itself; "FlashAttention v1～v4 完整进化史", v4 part 3 (lazy
    rescaling) lets the accumulator's reference lag the running maximum so
    that most tiles skip the rescale. Reading for fp8: the reference is the
    running maximum rounded up to a whole power of two (ln2 times an
    integer), which keeps P~ <= 1 so that P~ * 448 still fits e4m3, and
    makes every rescale factor a power of two; the GPU path then scales the
    product with V inside the matrix instruction and multiplies the
    accumulator only when the reference has moved far. Cost, measured with
    this oracle (same study, same 8 heads): RMSE of O 0.2358 against 0.2309
    with the exact running maximum (the maximum's own weight is no longer
    exactly 448 before rounding). reference="exact" keeps the plain
    running maximum for comparison.

Pins: tests/test_oracle_fp8.py (all 65,536 bf16 bit patterns against the
CPU library cast to float8_e4m3fn, hand-decoded codes, scale properties).
The tiled fp8 attention emulation follows the pages' steps (it is an
approximation, not a closed form); its pins are that with P left in float64 it
reduces to the exact oracle on the dequantised inputs under either reference,
that its per-tile P rounding stays within the e4m3 half-step bound, that the
reference does not change the LSE, a three-key example worked by hand for
each reference, and a closed-form rebuild of its weights (tests/fp8_bounds.py).

The backward of the fp8 forward is not described on the pages (they put fp8
in the forward only). Reading: the codes and scales are the inputs, so no
gradient flows through the rounding; the gradients are those of attention at
the dequantised Q, K, V, formed by the backward step of "6.1 FlashAttention
V1详解" (sections 6.1-6.2) from the fp8 forward's saved O and L. Pinned: with
the exact O and L of the dequantised inputs it is the exact backward.
"""

from __future__ import annotations

import numpy as np

__all__ = ["E4M3_MAX", "e4m3_decode", "e4m3_encode", "pow2_scale", "block_scales",
           "quantize", "dequantize", "fp8_attention_tiled", "fp8_backward"]

E4M3_MAX = 448.0
LN2 = float(np.log(2.0))
_MIN_NORMAL_EXP = -6          # 2^-6 is the smallest normal magnitude
_MANT_BITS = 3
_BIAS = 7


def e4m3_decode(codes) -> np.ndarray:
    """Decode e4m3fn codes (uint8) to float64 values."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m / 8.0 * 2.0 ** _MIN_NORMAL_EXP
    nor = (1.0 + m / 8.0) * np.exp2((e - _BIAS).astype(np.float64))
    val = np.where(e == 0, sub, nor) * sign
    return np.where((e == 0xF) & (m == 0x7), np.nan, val)


def e4m3_encode(x) -> np.ndarray:
    """Encode values to e4m3fn codes: saturate to +-448, then round to nearest even.

    NaN maps to 0x7F (sign kept). -0.0 keeps its sign bit.
    """
    with np.errstate(invalid="ignore"):
        x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, a)
    with np.errstate(divide="ignore"):
        ex = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    # log2 of values just below a power of two can round up; fix by checking.
    ex = np.where(np.exp2(ex) > a, ex - 1, ex)
    ex = np.where(np.exp2(ex + 1) <= a, ex + 1, ex)
    ex = np.maximum(ex, _MIN_NORMAL_EXP)
    step = np.exp2(ex - _MANT_BITS)              # spacing of representable values
    qv = np.rint(a / step) * step                # exact: step is a power of two
    qv = np.minimum(qv, E4M3_MAX)
    # Re-encode the rounded magnitude (rounding can carry into the next binade).
    with np.errstate(divide="ignore"):
        e2 = np.floor(np.log2(np.where(qv > 0, qv, 1.0)))
    e2 = np.where(np.exp2(e2) > qv, e2 - 1, e2)
    e2 = np.where(np.exp2(e2 + 1) <= qv, e2 + 1, e2)
    is_sub = (qv < 2.0 ** _MIN_NORMAL_EXP)
    mant_sub = np.rint(qv / 2.0 ** (_MIN_NORMAL_EXP - _MANT_BITS))
    mant_nor = np.rint((qv / np.exp2(e2) - 1.0) * 8.0)
    efield = np.where(is_sub, 0, e2 + _BIAS)
    mfield = np.where(is_sub, mant_sub, mant_nor)
    code = (efield.astype(np.int64) << 3) | mfield.astype(np.int64)
    code = np.where(qv == 0, 0, code)
    code = np.where(nan, 0x7F, code)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


def pow2_scale(r) -> np.ndarray:
    """Smallest power of two at or above r (r >= 0, float32 values), at least
    2^-126; 1 where r == 0. Returned as float32 (exact)."""
    r = np.asarray(r, dtype=np.float64)
    m, e = np.frexp(np.where(r > 0, r, 1.0))       # r = m 2^e, 0.5 <= m < 1
    s = np.where(m == 0.5, np.ldexp(1.0, e - 1), np.ldexp(1.0, e))
    s = np.maximum(s, 2.0 ** -126)
    return np.where(r > 0, s, 1.0).astype(np.float32)


def _scale_of(amax, pow2: bool) -> np.ndarray:
    """Scale of blocks with largest magnitudes amax (float32 array)."""
    amax = np.asarray(amax, dtype=np.float32)
    r = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    # a nonzero block whose amax / 448 underflows to 0 gets the smallest
    # positive float32 (2^-126 in the power-of-two form)
    r = np.where(amax > 0, np.maximum(r, np.float32(2.0 ** -149)), np.float32(0)).astype(np.float32)
    if pow2:
        return pow2_scale(r)
    return np.where(amax > 0, r, np.float32(1.0)).astype(np.float32)


def block_scales(x, block_rows: int, pow2: bool = False) -> np.ndarray:
    """Block scales in float32 for x of shape [B, H, N, d].

    s = float32(amax) / 448 rounded to float32 (1 for an all-zero block,
    2^-149 where that quotient underflows); with pow2, the smallest power of
    two at or above it, at least 2^-126 (1 for an all-zero block).
    block_rows > 0: one scale per block of ``block_rows`` rows of each
    (batch, head), shape [B, H, ceil(N / block_rows)]. block_rows == 0: one
    scale for the whole tensor, returned broadcast to shape [B, H, ceil(N/64)].
    """
    x = np.asarray(x, dtype=np.float32)
    B, H, N, _ = x.shape
    nb64 = -(-N // 64)
    if block_rows == 0:
        amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
        return np.full((B, H, nb64), _scale_of(amax, pow2), dtype=np.float32)
    nb = -(-N // block_rows)
    out = np.empty((B, H, nb), dtype=np.float32)
    for i in range(nb):
        blk = np.abs(x[:, :, i * block_rows:(i + 1) * block_rows, :])
        out[:, :, i] = _scale_of(blk.max(axis=(2, 3)).astype(np.float32), pow2)
    return out


def _expand_rows(s, N, block_rows):
    idx = np.arange(N) // block_rows
    return s[:, :, idx]


def quantize(x, block_rows: int, rot=None, pow2: bool = False):
    """Quantise x [B, H, N, d] to e4m3 codes with per-block scales
    (``block_scales``; pow2 selects the power-of-two form).

    With ``rot`` (d x d), x is first multiplied by it on the right, in
    float64, and the product rounded to float32 (the GPU forms it in float32
    in a different summation order; codes are compared with that in mind).
    The division x / s is taken in float32 (a quotient past 448 saturates).
    Returns (codes uint8, scales f32,
    the float32 values that were quantised).
    """
    x = np.asarray(x, dtype=np.float64)
    if rot is not None:
        x = x @ np.asarray(rot, dtype=np.float64)
    xf = x.astype(np.float32)
    s = block_scales(xf, block_rows, pow2)
    br = block_rows if block_rows > 0 else 64
    srow = _expand_rows(s, xf.shape[2], br)[..., None].astype(np.float32)
    y = (xf / srow).astype(np.float32)
    return e4m3_encode(y), s, xf


def dequantize(codes, scales, block_rows: int = 64) -> np.ndarray:
    """Dequantised float64 values: decode(code) * s of the code's row block."""
    c = np.asarray(codes)
    br = block_rows if block_rows > 0 else 64
    srow = _expand_rows(np.asarray(scales, dtype=np.float64), c.shape[2], br)[..., None]
    return e4m3_decode(c) * srow


def fp8_attention_tiled(q8, sq, k8, sk, v8, sv, scale: float, causal: bool,
                        B_c: int = 64, quantize_p: bool = True, block_rows: int = 64,
                        reference: str = "pow2"):
    """fp8 attention following the pages' tiled steps, in float64.

    Inputs are e4m3 codes with per-block scales. For each key tile of B_c
    keys: S = scale * Q K^T on the dequantised values, the online update of
    the row's reference m and sum, P~ = exp(S - m_new); the sum l uses P~
    itself while the product with V uses P~ rounded through e4m3 as
    e4m3(P~ * 448) / 448 (taken in float32, the precision the GPU forms P~
    in). O = sum / l at the end.

    reference = "exact": m is the running maximum of the row. reference =
    "pow2" (the lazy rescaling of "FlashAttention v1～v4 完整进化史", v4
    part 3, adapted to e4m3's range): m is kept on whole powers of two, the
    smallest at or above the running maximum (m in ln2 * Z); it moves, and
    the accumulator is rescaled by a power of two, only when a tile's maximum
    passes it, and P~ <= 1 still holds. Without the P rounding both give the
    exact attention.

    With quantize_p=False the P rounding is skipped and the result equals the
    exact attention of the dequantised inputs (a pin).
    Returns (O, LSE) float64, shapes [B, H, N, d] and [B, H, N].
    """
    if reference not in ("pow2", "exact"):
        raise ValueError(reference)
    qd = dequantize(q8, sq, block_rows)
    kd = dequantize(k8, sk, block_rows)
    vd = dequantize(v8, sv, block_rows)
    B, H, N, d = qd.shape
    o_all = np.zeros_like(qd)
    lse_all = np.empty((B, H, N))
    t_c = -(-N // B_c)
    for b in range(B):
        for h in range(H):
            q, k, v = qd[b, h], kd[b, h], vd[b, h]
            m = np.full(N, -np.inf)
            l = np.zeros(N)
            o = np.zeros((N, d))
            for j in range(t_c):
                c0, c1 = j * B_c, min(N, (j + 1) * B_c)
                s = scale * (q @ k[c0:c1].T)
                if causal:
                    s = np.where(np.arange(c0, c1)[None, :] > np.arange(N)[:, None], -np.inf, s)
                tmax = s.max(axis=1)
                if reference == "pow2":
                    with np.errstate(invalid="ignore"):
                        tmax = np.where(np.isfinite(tmax), np.ceil(tmax / LN2) * LN2, tmax)
                m_new = np.maximum(m, tmax)
                live = np.isfinite(m_new)
                m_ref = np.where(live, m_new, 0.0)
                alpha = np.where(live, np.exp(m - m_ref), 0.0)
                p = np.where(live[:, None], np.exp(s - m_ref[:, None]), 0.0)
                l = alpha * l + p.sum(axis=1)
                if quantize_p:
                    p32 = p.astype(np.float32) * np.float32(E4M3_MAX)
                    pv = e4m3_decode(e4m3_encode(p32)) / E4M3_MAX
                else:
                    pv = p
                o = alpha[:, None] * o + pv @ v[c0:c1]
                m = m_new
            o_all[b, h] = o / np.where(l > 0, l, 1.0)[:, None]
            lse_all[b, h] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o_all, lse_all


def fp8_backward(q8, sq, k8, sk, v8, sv, o, lse, do, scale: float, causal: bool, block_rows: int = 64):
    """Gradients (dQ, dK, dV, float64) with respect to the dequantised Q, K, V
    of the fp8 forward, from its saved O [B, H, N, d] and LSE [B, H, N] and
    the upstream gradient dO: the backward step on the saved statistics
    (P = exp(S - L) from the exact scores of the dequantised inputs, D =
    rowsum(dO * O)), applied to decode(code) * s.
    """
    from oracle import attention as A
    qd = dequantize(q8, sq, block_rows)
    kd = dequantize(k8, sk, block_rows)
    vd = dequantize(v8, sv, block_rows)
    return A.backward_from_saved(qd, kd, vd, o, lse, do, scale, causal)

"""Pins of the oracle's e4m3 codec, block quantiser and fp8 attention emulation."""

import numpy as np
import pytest

from oracle import attention as A
from oracle import fp8 as F
from seeded_inputs import bf16_bits_to_f32


def _torch():
    import torch
    return torch


def test_decode_all_codes_against_torch():
    torch = _torch()
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_decode(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    both_nan = np.isnan(ours) & np.isnan(theirs)
    assert np.all(both_nan | (ours == theirs))
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF]) and np.sum(np.isnan(ours)) == 2


def test_known_codes():
    assert F.e4m3_decode(np.uint8(0x7E)) == 448.0        # largest finite
    assert F.e4m3_decode(np.uint8(0x38)) == 1.0
    assert F.e4m3_decode(np.uint8(0x08)) == 2.0 ** -6    # smallest normal
    assert F.e4m3_decode(np.uint8(0x01)) == 2.0 ** -9    # smallest subnormal
    assert F.e4m3_decode(np.uint8(0xC0)) == -2.0
    assert F.e4m3_encode(np.array([448.0, 1e9, -1e9, 464.0, 0.0]))[:5].tolist() == \
        [0x7E, 0x7E, 0xFE, 0x7E, 0x00]


def test_encode_every_bf16_pattern_against_torch():
    """All 65,536 bf16 bit patterns, cast through float32, against torch's cast.

    torch's cast does not saturate (magnitudes from 464 up become NaN), so
    those inputs are checked against saturation to +-448 instead.
    """
    torch = _torch()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bf16_bits_to_f32(bits)
    ours = F.e4m3_encode(x)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    finite_small = np.isfinite(x) & (np.abs(x) < 464.0)
    assert np.array_equal(ours[finite_small], theirs[finite_small])
    big = np.isfinite(x) & (np.abs(x) >= 464.0)
    assert np.all((ours[big] & 0x7F) == 0x7E)
    assert np.all((ours[big] >> 7) == (x[big] < 0))
    nan = np.isnan(x)
    assert np.all((ours[nan] & 0x7F) == 0x7F)
    inf = np.isinf(x)
    assert np.all((ours[inf] & 0x7F) == 0x7E)


def test_roundtrip_error_is_half_step():
    rng = np.random.default_rng(31)
    x = rng.standard_normal(100000) * 50
    x = np.clip(x, -448, 448)
    y = F.e4m3_decode(F.e4m3_encode(x))
    a = np.abs(x)
    ex = np.maximum(np.floor(np.log2(np.maximum(a, 1e-300))), -6)
    half_step = np.exp2(ex - 3) / 2
    assert np.all(np.abs(y - x) <= half_step * (1 + 1e-12))


@pytest.mark.parametrize("pow2", [False, True])
def test_block_scales_and_codes(pow2):
    rng = np.random.default_rng(32)
    x = rng.standard_normal((2, 3, 150, 16)).astype(np.float32)
    x[1, 2, 64:128] = 0.0
    codes, s, xf = F.quantize(x, 64, pow2=pow2)
    assert s.shape == (2, 3, 3)
    assert s[1, 2, 1] == 1.0
    for b in range(2):
        for h in range(3):
            for i in range(3):
                blk = xf[b, h, 64 * i:64 * (i + 1)]
                amax = np.float32(np.abs(blk).max())
                if amax > 0:
                    r = np.float64(np.float32(amax / np.float32(448.0)))
                    si = np.float64(s[b, h, i])
                    cblk = codes[b, h, 64 * i:64 * (i + 1)]
                    if pow2:
                        # a power of two, the smallest at or above amax / 448
                        assert np.frexp(si)[0] == 0.5
                        assert r <= si < 2 * r
                        # the largest element lands in (224, 448]: codes 0x76 .. 0x7E
                        assert 0x76 <= np.max(cblk & 0x7F) <= 0x7E
                    else:
                        # amax / 448 itself: the largest element gets the top code
                        assert si == r
                        assert np.max(cblk & 0x7F) == 0x7E
    d = F.dequantize(codes, s, 64)
    srow = s[:, :, np.arange(150) // 64][..., None]
    assert np.all(np.abs(d - x) <= srow * 448 * 2.0 ** -4 + 1e-30)
    # per-tensor: one scale everywhere
    c0, s0, _ = F.quantize(x, 0, pow2=pow2)
    assert np.all(s0 == s0.flat[0])
    r0 = np.float64(np.float32(np.float32(np.abs(x).max()) / np.float32(448)))
    if pow2:
        assert np.frexp(np.float64(s0.flat[0]))[0] == 0.5 and r0 <= s0.flat[0] < 2 * r0
    else:
        assert s0.flat[0] == r0


def test_block_scale_edge_cases():
    """All-zero blocks get 1; a block whose amax / 448 underflows gets the
    smallest positive float32 (2^-126 in the power-of-two form), so nonzero
    elements still get nonzero codes and zeros stay zero."""
    x = np.zeros((1, 1, 128, 4), np.float32)
    x[0, 0, 64, 0] = np.float32(2.0 ** -148)       # amax / 448 underflows
    x[0, 0, 65, 1] = -np.float32(2.0 ** -149)
    c, s, _ = F.quantize(x, 64)
    assert s[0, 0, 0] == 1.0 and s[0, 0, 1] == np.float32(2.0 ** -149)
    assert np.all(c[0, 0, :64] == 0)
    assert c[0, 0, 64, 0] != 0 and c[0, 0, 65, 1] & 0x7F != 0 and c[0, 0, 65, 1] & 0x80
    assert np.all(c[0, 0, 64, 1:] == 0)
    c2, s2, _ = F.quantize(x, 64, pow2=True)
    assert s2[0, 0, 0] == 1.0 and s2[0, 0, 1] == np.float32(2.0 ** -126)


def test_pow2_scale():
    """The block scale is the smallest power of two at or above its argument
    (an exact power of two is kept), at least 2^-126, and 1 for zero."""
    rng = np.random.default_rng(34)
    r = np.concatenate([np.exp2(rng.uniform(-140, 120, 5000)), np.exp2(np.arange(-126, 120, 7.0)),
                        np.nextafter(np.exp2(np.arange(-100, 100, 9.0)), 0), [0.0, 2.0 ** -149, 2.0 ** -127]])
    r = r.astype(np.float32).astype(np.float64)
    s = F.pow2_scale(r).astype(np.float64)
    pos = r > 0
    assert np.all(s[~pos] == 1.0)
    assert np.all(np.frexp(s[pos])[0] == 0.5)                  # powers of two
    assert np.all(s[pos] >= np.maximum(r[pos], 2.0 ** -126))
    big = r > 2.0 ** -126
    assert np.all(s[big] < 2 * r[big])                          # the smallest such
    assert np.all(s[pos & ~big] == 2.0 ** -126)
    exact = np.exp2(np.arange(-126, 120, 7.0))
    assert np.all(F.pow2_scale(exact) == exact)


def test_rotation_leaves_scores_unchanged_before_rounding():
    rng = np.random.default_rng(33)
    d = 16
    m, _ = np.linalg.qr(rng.standard_normal((d, d)))
    q = rng.standard_normal((1, 1, 64, d))
    k = rng.standard_normal((1, 1, 64, d))
    _, _, qr_ = F.quantize(q, 64, rot=m)
    _, _, kr_ = F.quantize(k, 64, rot=m)
    s1 = qr_[0, 0].astype(np.float64) @ kr_[0, 0].astype(np.float64).T
    s2 = q[0, 0] @ k[0, 0].T
    assert np.max(np.abs(s1 - s2)) <= 1e-4


@pytest.mark.parametrize("reference", ["pow2", "exact"])
def test_fp8_emulation_without_p_rounding_is_exact_attention(reference):
    rng = np.random.default_rng(34)
    x = {n: rng.standard_normal((1, 2, 130, 16)) for n in "qkv"}
    qc = {n: F.quantize(x[n], 64) for n in "qkv"}
    for causal in (False, True):
        o, lse = F.fp8_attention_tiled(qc["q"][0], qc["q"][1], qc["k"][0], qc["k"][1],
                                       qc["v"][0], qc["v"][1], 0.25, causal, B_c=64,
                                       quantize_p=False, reference=reference)
        deq = {n: F.dequantize(qc[n][0], qc[n][1], 64) for n in "qkv"}
        o_ref, l_ref = A.forward(deq["q"], deq["k"], deq["v"], 0.25, causal)
        assert np.max(np.abs(o - o_ref)) <= 1e-12
        assert np.max(np.abs(lse - l_ref)) <= 1e-12


@pytest.mark.parametrize("reference", ["pow2", "exact"])
def test_fp8_emulation_p_rounding_within_bound(reference):
    """Rounding P~ * 448 to e4m3 moves each weight by at most half a step.

    |P8 - P~| <= 2^-4 P~ + 2^-10 / 448 per weight, so each O element moves by
    at most (2^-4 + 2^-10 / 448 * n_keys / l) * max|v|, where l, the sum of
    P~ in the units of the final reference, is at least the maximum's own
    P~: 1 with the exact maximum, at least 1/2 with the power-of-two
    reference. The V rows are scaled per block so that the V block scales
    differ.
    """
    rng = np.random.default_rng(35)
    x = {n: rng.standard_normal((1, 1, 192, 16)) for n in "qkv"}
    x["v"] *= np.repeat(np.array([1.0, 6.0, 0.5]), 64)[None, None, :, None]
    qc = {n: F.quantize(x[n], 64) for n in "qkv"}
    args = (qc["q"][0], qc["q"][1], qc["k"][0], qc["k"][1], qc["v"][0], qc["v"][1], 0.25, False)
    o8, l8 = F.fp8_attention_tiled(*args, B_c=64, quantize_p=True, reference=reference)
    o, l = F.fp8_attention_tiled(*args, B_c=64, quantize_p=False, reference=reference)
    vmax = np.abs(F.dequantize(qc["v"][0], qc["v"][1], 64)).max()
    l_min = 1.0 if reference == "exact" else 0.5
    bound = (2.0 ** -4 + 2.0 ** -10 / 448 * 192 / l_min) * vmax
    assert np.max(np.abs(o8 - o)) <= bound
    assert np.max(np.abs(o8 - o)) > 0          # the rounding is really applied
    assert np.array_equal(l8, l)                # l comes from the unrounded P~


@pytest.mark.parametrize("reference", ["pow2", "exact"])
def test_fp8_emulation_v_scale_power_of_two_invariance(reference):
    """Multiplying every V block scale by 2^k (same codes) multiplies O by 2^k exactly.

    P and its e4m3 codes do not depend on V, so only the dequantised V is
    scaled, and by a power of two that rounds nothing.
    """
    rng = np.random.default_rng(36)
    x = {n: rng.standard_normal((1, 2, 150, 8)) for n in "qkv"}
    x["v"][:, :, 64:128] *= 0.1
    qc = {n: F.quantize(x[n], 64) for n in "qkv"}
    for causal in (False, True):
        base = (qc["q"][0], qc["q"][1], qc["k"][0], qc["k"][1], qc["v"][0])
        o1, l1 = F.fp8_attention_tiled(*base, qc["v"][1], 0.3, causal, reference=reference)
        o2, l2 = F.fp8_attention_tiled(*base, qc["v"][1] * np.float32(8.0), 0.3, causal, reference=reference)
        assert np.array_equal(o2, 8.0 * o1)
        assert np.array_equal(l2, l1)


@pytest.mark.parametrize("reference", ["pow2", "exact"])
def test_bound_helper_rebuilds_the_emulation(reference):
    """tests/fp8_bounds.py rebuilds the emulation's O in closed form (each key's
    weight from the reference in force at its tile, no running rescale); the
    online emulation must agree."""
    import sys, os
    sys.path.insert(0, os.path.dirname(__file__))
    from fp8_bounds import bound_rows
    rng = np.random.default_rng(37)
    x = {n: rng.standard_normal((1, 1, 200, 16)) for n in "qkv"}
    x["v"] *= np.repeat(np.array([1.0, 4.0, 0.3, 2.0]), 64)[None, None, :200, None]
    qc = {n: F.quantize(x[n], 64) for n in "qkv"}
    for causal in (False, True):
        o, lse = F.fp8_attention_tiled(qc["q"][0], qc["q"][1], qc["k"][0], qc["k"][1],
                                       qc["v"][0], qc["v"][1], 0.25, causal, reference=reference)
        rows = np.arange(200)
        _, _, o_em, l_em = bound_rows(qc["q"][0][0, 0], qc["q"][1][0, 0], qc["k"][0][0, 0], qc["k"][1][0, 0],
                                      qc["v"][0][0, 0], qc["v"][1][0, 0], 0.25, causal, rows,
                                      reference=reference)
        assert np.max(np.abs(o_em - o[0, 0])) <= 1e-12
        assert np.max(np.abs(l_em - lse[0, 0])) <= 1e-12


def _hand_example(reference):
    q8 = F.e4m3_encode(np.ones(3)).reshape(1, 1, 3, 1)      # three equal query rows
    k8 = F.e4m3_encode(np.array([0.5, 2.0, 1.125])).reshape(1, 1, 3, 1)
    v8 = F.e4m3_encode(np.array([1.0, -2.0, 0.5])).reshape(1, 1, 3, 1)
    unit = np.ones((1, 1, 1), dtype=np.float32)
    return F.fp8_attention_tiled(q8, unit, k8, unit, v8, unit, 1.0, False, B_c=1, reference=reference)


def test_fp8_emulation_hand_example_power_of_two_reference():
    """Queries all 1 (three equal rows), keys 0.5, 2.0, 1.125 (scores equal to them), values
    1, -2, 0.5, one key per tile, worked by hand.

    In log2 units the scores are 0.7213, 2.8854, 1.6231. The reference after
    each tile is the running maximum rounded up to an integer: 1, 3, 3. P' =
    448 * 2^(score - reference) = 369.31, 413.79, 172.49, whose nearest e4m3
    values are 384, 416 and 176 (steps of 32 above 256, of 16 below). A key
    weighs code * 2^reference / 448 against the unrounded denominator
    e^0.5 + e^2 + e^1.125, so O = (768 - 6656 + 704) / 448 / (e^0.5 + e^2 +
    e^1.125), and LSE is the log of that denominator.
    """
    o, lse = _hand_example("pow2")
    den = np.exp(0.5) + np.exp(2.0) + np.exp(1.125)
    assert np.max(np.abs(o[0, 0, :, 0] - (384 * 2 * 1.0 + 416 * 8 * -2.0 + 176 * 8 * 0.5) / 448 / den)) <= 1e-14
    assert np.max(np.abs(lse[0, 0] - np.log(den))) <= 1e-14


def test_fp8_emulation_hand_example_exact_reference():
    """The same example with the exact running maximum: the first two keys are
    each their tile's maximum, so P' = 448 exactly, and the third has P' =
    448 e^(1.125 - 2) = 186.75, nearest e4m3 value 192; the earlier keys are
    rescaled in float64 without rounding."""
    o, lse = _hand_example("exact")
    den = np.exp(0.5) + np.exp(2.0) + np.exp(1.125)
    num = np.exp(0.5) * 1.0 + np.exp(2.0) * -2.0 + 192 / 448 * np.exp(2.0) * 0.5
    assert np.max(np.abs(o[0, 0, :, 0] - num / den)) <= 1e-14
    assert np.max(np.abs(lse[0, 0] - np.log(den))) <= 1e-14


def test_fp8_reference_leaves_the_lse_unchanged():
    """The row sum is kept in the units of whichever reference is in force and
    rescaled exactly with it, so the LSE is the same for both references (and
    equals that of the dequantised inputs); O differs only by P's rounding."""
    rng = np.random.default_rng(39)
    x = {n: rng.standard_normal((1, 2, 150, 16)) * 2.0 for n in "qkv"}
    qc = {n: F.quantize(x[n], 64) for n in "qkv"}
    args = (qc["q"][0], qc["q"][1], qc["k"][0], qc["k"][1], qc["v"][0], qc["v"][1], 0.25)
    deq = {n: F.dequantize(qc[n][0], qc[n][1], 64) for n in "qkv"}
    for causal in (False, True):
        o1, l1 = F.fp8_attention_tiled(*args, causal, reference="pow2")
        o2, l2 = F.fp8_attention_tiled(*args, causal, reference="exact")
        _, l_ref = A.forward(deq["q"], deq["k"], deq["v"], 0.25, causal)
        assert np.max(np.abs(l1 - l2)) <= 1e-12 and np.max(np.abs(l1 - l_ref)) <= 1e-12
        assert np.max(np.abs(o1 - o2)) > 0


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_backward_with_exact_statistics_is_the_exact_backward(causal):
    """Given the exact O and L of the dequantised inputs, the fp8 backward is
    the exact backward of attention at those inputs (A.backward recomputes
    everything itself, blockwise, and shares no step with the saved-statistics
    path but the definitions)."""
    rng = np.random.default_rng(38)
    x = {n: rng.standard_normal((1, 2, 150, 16)) for n in "qkv"}
    x["k"][:, :, 70:80] *= 6.0
    do = rng.standard_normal((1, 2, 150, 16))
    qc = {n: F.quantize(x[n], 64, pow2=True) for n in "qkv"}
    deq = {n: F.dequantize(qc[n][0], qc[n][1], 64) for n in "qkv"}
    o, lse = A.forward(deq["q"], deq["k"], deq["v"], 0.25, causal)
    got = F.fp8_backward(qc["q"][0], qc["q"][1], qc["k"][0], qc["k"][1], qc["v"][0], qc["v"][1],
                         o, lse, do, 0.25, causal)
    ref = A.backward(deq["q"], deq["k"], deq["v"], do, 0.25, causal)
    for g, r in zip(got, ref):
        assert np.max(np.abs(g - r)) <= 1e-10 * max(1.0, np.max(np.abs(r)))


def test_fp8_backward_follows_the_saved_output():
    """D = rowsum(dO * O) uses the given O: moving O by e along dO moves dQ
    and dK by exactly the linear term and leaves dV alone."""
    rng = np.random.default_rng(39)
    x = {n: rng.standard_normal((1, 1, 96, 8)) for n in "qkv"}
    do = rng.standard_normal((1, 1, 96, 8))
    qc = {n: F.quantize(x[n], 64, pow2=True) for n in "qkv"}
    deq = {n: F.dequantize(qc[n][0], qc[n][1], 64) for n in "qkv"}
    o, lse = A.forward(deq["q"], deq["k"], deq["v"], 0.3, False)
    args = (qc["q"][0], qc["q"][1], qc["k"][0], qc["k"][1], qc["v"][0], qc["v"][1])
    g0 = F.fp8_backward(*args, o, lse, do, 0.3, False)
    e = 1e-3
    g1 = F.fp8_backward(*args, o + e * do, lse, do, 0.3, False)
    assert np.array_equal(g0[2], g1[2])
    # D grows by e * rowsum(dO^2); dS by -P * that; dQ by -scale * e * (P * rowsum) K
    s = 0.3 * deq["q"][0, 0] @ deq["k"][0, 0].T
    p = np.exp(s - lse[0, 0][:, None])
    r = np.sum(do[0, 0] ** 2, axis=1)
    ddq = -0.3 * e * (p * r[:, None]) @ deq["k"][0, 0]
    ddk = -0.3 * e * (p * r[:, None]).T @ deq["q"][0, 0]
    assert np.max(np.abs((g1[0] - g0[0])[0, 0] - ddq)) <= 1e-12
    assert np.max(np.abs((g1[1] - g0[1])[0, 0] - ddk)) <= 1e-12

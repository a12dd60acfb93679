"""The seeded input generators: bf16 rounding, determinism, outliers, rotation."""

import numpy as np

import seeded_inputs as si


def test_bf16_round_matches_torch():
    import torch
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        # exact ties between two bf16 values, both parities
                        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
                        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, 1e-40], dtype=np.float32)])
    bits, vals = si.bf16_round(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, want)
    assert np.array_equal(vals.view(np.uint32) >> 16, bits.astype(np.uint32))


def test_inputs_are_deterministic_and_order_independent():
    w = si.workload(3).resized(B=1, H=2, N=40)
    a = si.make_inputs(w)
    b = si.make_inputs(w, names=("v",))
    assert np.array_equal(a["v_bits"], b["v_bits"])
    assert not np.array_equal(a["q_bits"], a["k_bits"])
    c = si.make_inputs(w)
    for n in "qkv":
        assert np.array_equal(a[n + "_bits"], c[n + "_bits"])


def test_fp8_workload_outliers_and_rotation():
    w = si.workload(5)
    small = w.resized(B=1, N=70)
    x = si.make_inputs(small, names=("q", "k", "v"))
    assert x["outliers"].shape == (4, 2)          # round(0.001 * 32 * 128) = 4 channels
    m = x["rot"].astype(np.float64)
    assert np.max(np.abs(m @ m.T - np.eye(w.d))) <= 1e-6
    # the outlier channels are the only ones with large magnitudes
    for hh, dd in x["outliers"]:
        assert np.abs(x["q"][0, hh, :, dd]).max() > 10


def test_haar_is_orthogonal_and_seeded():
    m1 = si.haar_orthogonal(np.random.default_rng(5), 16)
    m2 = si.haar_orthogonal(np.random.default_rng(5), 16)
    assert np.array_equal(m1, m2)
    assert np.max(np.abs(m1.T @ m1 - np.eye(16))) <= 1e-12

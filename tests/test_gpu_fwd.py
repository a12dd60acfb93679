"""Forward parity on the GPU: the HIP kernels against the float64 oracle.

Tolerances (stated with the workloads): float32 inputs, max-abs 1e-5 on O and
LSE; bf16 inputs, max-abs 2e-2 on O (bf16) and 1e-3 on LSE (float32).
Small shapes are compared element by element over the whole output; the
full-size workloads over whole sampled heads plus rows sampled across every
head (each row from its full score row).
"""

import math

import numpy as np
import pytest

import seeded_inputs as si
from gpu_util import announce, bf16_from_f32, dev_tensor, host, max_abs
from oracle import attention as A

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 1e-3)}


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import exact_tiled_attention_12_amd as m
    m.load()
    return m


def _run(fa, x, w, causal=None, scale=None):
    q, k, v = (dev_tensor(x, n, w.dtype) for n in "qkv")
    causal = w.causal if causal is None else causal
    announce(f"fa_fwd {w.dtype} B={w.B} H={w.H} N={w.N} d={w.d} causal={causal}")
    o, lse = fa.fwd(q, k, v, causal=causal, scale=w.scale if scale is None else scale)
    import torch
    torch.cuda.synchronize()
    return host(o), host(lse)


def _compare_full(fa, w, causal=None):
    x = si.make_inputs(w, names=("q", "k", "v"))
    o, lse = _run(fa, x, w, causal)
    c = w.causal if causal is None else causal
    o_ref, l_ref = A.forward(x["q"], x["k"], x["v"], w.scale, c)
    to, tl = TOL[w.dtype]
    eo, el = max_abs(o, o_ref), max_abs(lse, l_ref)
    assert eo <= to, f"O max-abs {eo:.3e} > {to}"
    assert el <= tl, f"LSE max-abs {el:.3e} > {tl}"
    return eo, el


def test_workload1_fp32_full(fa):
    eo, el = _compare_full(fa, si.workload(1))
    print(f"workload 1: O {eo:.2e} LSE {el:.2e}")


def test_workload2_bf16_full(fa):
    eo, el = _compare_full(fa, si.workload(2))
    print(f"workload 2: O {eo:.2e} LSE {el:.2e}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 63, 64, 65, 127, 129, 200, 257])
def test_ragged_shapes(fa, dtype, d, causal, N):
    w = si.Workload(900 + N, "ragged", 2, 3, N, d, dtype, causal, False)
    _compare_full(fa, w)


def _sampled(fa, w, heads, n_rows):
    x = si.make_inputs(w, names=("q", "k", "v"))
    o, lse = _run(fa, x, w)
    to, tl = TOL[w.dtype]
    worst_o = worst_l = 0.0
    for (b, h) in heads:
        o_ref, l_ref = A.forward(x["q"][b, h], x["k"][b, h], x["v"][b, h], w.scale, w.causal)
        worst_o = max(worst_o, max_abs(o[b, h], o_ref))
        worst_l = max(worst_l, max_abs(lse[b, h], l_ref))
    rng = np.random.default_rng(77)
    for _ in range(n_rows // 16):
        b, h = int(rng.integers(w.B)), int(rng.integers(w.H))
        rows = rng.choice(w.N, size=16, replace=False)
        rows[0] = w.N - 1
        o_ref, l_ref = A.forward_rows(x["q"][b, h], x["k"][b, h], x["v"][b, h], rows, w.scale, w.causal)
        worst_o = max(worst_o, max_abs(o[b, h][rows], o_ref))
        worst_l = max(worst_l, max_abs(lse[b, h][rows], l_ref))
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    print(f"{w.name}: O {worst_o:.2e} LSE {worst_l:.2e}")
    assert worst_o <= to and worst_l <= tl, (worst_o, worst_l)


def test_workload3_sampled(fa):
    w = si.workload(3)
    _sampled(fa, w, heads=[(0, 0), (1, 31), (0, 17)], n_rows=256)


def test_workload4_forward_sampled(fa):
    w = si.workload(4)
    _sampled(fa, w, heads=[(0, 5), (0, 30)], n_rows=256)


def test_worked_example_on_gpu(fa):
    """Scores [1, 2, 0, 3] for every query ("FlashAttention v1～v4 完整进化史", v1 part 2).

    q = e0, k_j = x_j e0, v_j = e_j, scale 1: row i of O holds the softmax of
    [1, 2, 0, 3] in its first four columns and LSE = 3 + ln(l2) with
    l2 = e^-2 + e^-1 + e^-3 + 1.
    """
    import torch
    x = np.array([1.0, 2.0, 0.0, 3.0])
    d, N = 64, 4
    q = np.zeros((1, 1, N, d), np.float32); q[..., 0] = 1.0
    k = np.zeros((1, 1, N, d), np.float32); k[0, 0, :, 0] = x
    v = np.zeros((1, 1, N, d), np.float32)
    for j in range(N):
        v[0, 0, j, j] = 1.0
    l2 = math.exp(-2) + math.exp(-1) + math.exp(-3) + 1
    want = np.exp(x - 3) / l2
    for dt in ("bf16", "f32"):
        if dt == "bf16":
            tq, tk, tv = (bf16_from_f32(a)[0] for a in (q, k, v))
        else:
            tq, tk, tv = (torch.from_numpy(a).cuda() for a in (q, k, v))
        announce(f"fa_fwd worked example {dt}")
        o, lse = fa.fwd(tq, tk, tv, causal=False, scale=1.0)
        o, lse = host(o), host(lse)
        tol = 2.0 ** -8 if dt == "bf16" else 1e-6
        assert np.max(np.abs(o[0, 0, :, :4] - want[None, :])) <= tol
        assert np.max(np.abs(o[0, 0, :, 4:])) == 0.0
        assert np.max(np.abs(lse - (3 + math.log(l2)))) <= 1e-6


def test_invariants_without_oracle(fa):
    """Causal row 0 is V_0 exactly; key permutation; bitwise re-runs; scale 0."""
    import torch
    w = si.Workload(950, "invariants", 2, 4, 300, 128, "bf16", True, False)
    x = si.make_inputs(w, names=("q", "k", "v"))
    q, k, v = (dev_tensor(x, n, "bf16") for n in "qkv")
    announce("fa_fwd invariants causal")
    o1, l1 = fa.fwd(q, k, v, causal=True)
    o2, l2 = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    assert torch.equal(o1[:, :, 0].view(torch.int16), v[:, :, 0].view(torch.int16))
    s0 = (x["q"][:, :, 0].astype(np.float64) * x["k"][:, :, 0]).sum(-1) * w.scale
    assert max_abs(host(l1)[:, :, 0], s0) <= 1e-5
    # key permutation leaves the non-causal output unchanged (up to fp32 summation order)
    perm = torch.randperm(w.N, generator=torch.Generator().manual_seed(3)).cuda()
    announce("fa_fwd invariants permuted keys")
    o3, l3 = fa.fwd(q, k, v, causal=False)
    o4, l4 = fa.fwd(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), causal=False)
    torch.cuda.synchronize()
    assert max_abs(host(o3), host(o4)) <= 2e-2 and max_abs(host(l3), host(l4)) <= 1e-4
    # scale 0: uniform weights, O = mean of V (prefix means when causal), LSE = ln(#keys)
    announce("fa_fwd invariants scale 0")
    o5, l5 = fa.fwd(q, k, v, causal=True, scale=0.0)
    vv = x["v"].astype(np.float64)
    pref = np.cumsum(vv, axis=2) / np.arange(1, w.N + 1)[None, None, :, None]
    assert max_abs(host(o5), pref) <= 1e-2
    assert max_abs(host(l5), np.log(np.arange(1, w.N + 1))[None, None, :]) <= 1e-5


def test_nan_propagates_to_its_row_only(fa):
    import torch
    w = si.Workload(951, "nan", 1, 2, 130, 64, "bf16", False, False)
    x = si.make_inputs(w, names=("q", "k", "v"))
    q, k, v = (dev_tensor(x, n, "bf16") for n in "qkv")
    q[0, 1, 7, 3] = float("nan")
    announce("fa_fwd nan row")
    o, lse = fa.fwd(q, k, v)
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    assert np.all(np.isnan(o[0, 1, 7])) and np.isnan(lse[0, 1, 7])
    o[0, 1, 7] = 0
    lse[0, 1, 7] = 0
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))

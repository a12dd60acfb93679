"""Fixed-order (deterministic) backward on the GPU: parity with the float64
oracle, bit-identical results across runs, and agreement with fa_bwd.

fa_bwd_det ("FlashAttention v1～v4 完整进化史", v4 part 4: the backward can
reduce dQ across workgroups in a fixed order) computes what fa_bwd computes;
only the order of the float32 dQ sum over key tiles is fixed. Tolerances are
those of the bf16 backward: every element within max(2e-2, one bf16 spacing
at |ref|).
"""

import numpy as np
import pytest

import seeded_inputs as si
from gpu_util import announce, bf16_ulp, dev_tensor, host, max_abs
from oracle import attention as A

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import exact_tiled_attention_12_amd as m
    m.load()
    return m


def _inputs(w):
    x = si.make_inputs(w)
    return x, [dev_tensor(x, n, "bf16") for n in ("q", "k", "v", "do")]


def _bits(t):
    import torch
    return t.view(torch.int16)


def _check(got, ref, what):
    for n, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert np.all(np.isfinite(g)), f"{what} {n} not finite"
        bound = np.maximum(2e-2, bf16_ulp(r))
        assert np.all(np.abs(g - r) <= bound), f"{what} {n}: max-abs {max_abs(g, r):.3e}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 65, 255, 257, 600])
def test_det_parity_ragged(fa, d, causal, N):
    import torch
    w = si.Workload(1200 + N, "bwd det bf16", 2, 3, N, d, "bf16", causal, True)
    x, (q, k, v, do) = _inputs(w)
    announce(f"fa_bwd_det B=2 H=3 N={N} d={d} causal={causal}")
    o, lse = fa.fwd(q, k, v, causal=causal, scale=w.scale)
    g = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=w.scale, deterministic=True)
    torch.cuda.synchronize()
    ref = A.backward(x["q"], x["k"], x["v"], x["do"], w.scale, causal)
    _check([host(t) for t in g], ref, f"det N={N} d={d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_det_bit_identical_runs_and_matches_fa_bwd(fa, d, causal):
    """Three runs give the same bits; dK and dV are fa_bwd's bits; dQ agrees
    with fa_bwd's to the rounding of a reordered float32 sum (both are
    rounded to bf16 once)."""
    import torch
    N = 1100   # 5 key tiles, 35 query tiles, ragged
    w = si.Workload(1300 + d, "bwd det runs", 1, 4, N, d, "bf16", causal, True)
    x, (q, k, v, do) = _inputs(w)
    announce(f"fa_bwd_det repeat N={N} d={d} causal={causal}")
    o, lse = fa.fwd(q, k, v, causal=causal)
    runs = [fa.bwd(q, k, v, o, lse, do, causal=causal, deterministic=True) for _ in range(3)]
    plain = fa.bwd(q, k, v, o, lse, do, causal=causal)
    torch.cuda.synchronize()
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(_bits(a), _bits(b))
    assert torch.equal(_bits(runs[0][1]), _bits(plain[1]))
    assert torch.equal(_bits(runs[0][2]), _bits(plain[2]))
    dq_det, dq_plain = host(runs[0][0]), host(plain[0])
    assert np.all(np.abs(dq_det - dq_plain) <= 2 * bf16_ulp(dq_plain) + 1e-6)


def test_det_workspace_reuse_with_garbage(fa):
    """The workspace needs no clearing: a buffer full of NaN gives the same bits."""
    import torch
    N, d = 700, 128
    w = si.Workload(1400, "bwd det ws", 1, 2, N, d, "bf16", True, True)
    x, (q, k, v, do) = _inputs(w)
    announce("fa_bwd_det workspace reuse")
    o, lse = fa.fwd(q, k, v, causal=True)
    need = fa.bwd_det_workspace_bytes(1, 2, N, d, True)
    ws = torch.empty(need, device="cuda", dtype=torch.uint8)
    a = fa.bwd(q, k, v, o, lse, do, causal=True, workspace=ws, deterministic=True)
    ws.view(torch.float32)[: need // 4].fill_(float("nan"))
    b = fa.bwd(q, k, v, o, lse, do, causal=True, workspace=ws, deterministic=True)
    torch.cuda.synchronize()
    for t1, t2 in zip(a, b):
        assert torch.equal(_bits(t1), _bits(t2))


def test_det_workload4_sampled_head_and_repeat(fa):
    """Full-size long-context workload (B=1, H=32, N=16384, d=128, causal):
    one whole head against the oracle, and two runs bit-identical."""
    import torch
    w = si.workload(4)
    x, (q, k, v, do) = _inputs(w)
    announce("fa_bwd_det workload 4")
    o, lse = fa.fwd(q, k, v, causal=True)
    ws = torch.empty(fa.bwd_det_workspace_bytes(w.B, w.H, w.N, w.d, True), device="cuda", dtype=torch.uint8)
    g1 = fa.bwd(q, k, v, o, lse, do, causal=True, workspace=ws, deterministic=True)
    g1 = [t.clone() for t in g1]
    g2 = fa.bwd(q, k, v, o, lse, do, causal=True, workspace=ws, deterministic=True)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(_bits(a), _bits(b))
    h = 17
    ref = A.backward_head(x["q"][0, h], x["k"][0, h], x["v"][0, h], x["do"][0, h], w.scale, True)
    _check([host(t)[0, h] for t in g1], ref, "det workload 4 head 17")

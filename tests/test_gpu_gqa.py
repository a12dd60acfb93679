"""Grouped-query (GQA) and multi-query (MQA) attention on the GPU against the
float64 oracle (oracle.attention.forward_gqa / backward_gqa).

Inputs: the seeded bf16 workload tensors of H heads; K and V keep their first
H_kv heads. Tolerances are the bf16 ones of the plain forward and backward
(O within 2e-2, LSE within 1e-3; gradients within max(2e-2, one bf16 spacing
at |ref|)). dK and dV of a shared head sum G query heads, so their |ref| grows
with G; the bound scales with it through the bf16 spacing term.
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


def _inputs(seed, B, H, H_kv, N, d, causal):
    w = si.Workload(seed, "gqa bf16", B, H, N, d, "bf16", causal, True)
    x = si.make_inputs(w)
    for n in ("k", "v"):
        x[n] = np.ascontiguousarray(x[n][:, :H_kv])
        x[n + "_bits"] = np.ascontiguousarray(x[n + "_bits"][:, :H_kv])
    return w, x, [dev_tensor(x, n, "bf16") for n in ("q", "k", "v", "do")]


def _check_grads(got, ref, what):
    for n, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert np.all(np.isfinite(g)), f"{what} {n} not finite"
        bound = np.maximum(2e-2, bf16_ulp(r))
        assert np.all(np.abs(g - r) <= bound), f"{what} {n}: max-abs {max_abs(g, r):.3e}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,H_kv", [(4, 2), (6, 1), (8, 2)])
@pytest.mark.parametrize("N", [1, 65, 257, 600])
def test_gqa_forward_backward_parity(fa, d, causal, H, H_kv, N):
    import torch
    w, x, (q, k, v, do) = _inputs(1500 + N + H, 2, H, H_kv, N, d, causal)
    announce(f"fa_fwd_gqa/fa_bwd_gqa B=2 H={H} H_kv={H_kv} N={N} d={d} causal={causal}")
    o, lse = fa.fwd(q, k, v, causal=causal, scale=w.scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    assert tuple(dk.shape) == (2, H_kv, N, d)
    o_ref, lse_ref = A.forward_gqa(x["q"], x["k"], x["v"], w.scale, causal)
    assert max_abs(host(o), o_ref) <= 2e-2
    assert max_abs(host(lse), lse_ref) <= 1e-3
    ref = A.backward_gqa(x["q"], x["k"], x["v"], x["do"], w.scale, causal)
    _check_grads([host(t) for t in (dq, dk, dv)], ref, f"gqa H={H}/{H_kv} N={N} d={d} causal={causal}")


def test_gqa_with_one_group_per_head_is_mha(fa):
    """fa_fwd_gqa / fa_bwd_gqa with H_kv = H give the bits of fa_fwd / fa_bwd
    (dQ up to its float32 atomic order)."""
    import torch
    from exact_tiled_attention_12_amd import _lib
    B, H, N, d = 1, 4, 300, 128
    w, x, (q, k, v, do) = _inputs(1600, B, H, H, N, d, True)
    announce("fa_fwd_gqa with H_kv = H")
    lib = _lib.load()
    st = torch.cuda.current_stream().cuda_stream
    o1, l1 = fa.fwd(q, k, v, causal=True)
    o2, l2 = torch.empty_like(q), torch.empty_like(l1)
    assert lib.fa_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), l2.data_ptr(),
                          B, H, H, N, d, w.scale, 1, st) == 0
    g1 = fa.bwd(q, k, v, o1, l1, do, causal=True)
    g2 = [torch.empty_like(q) for _ in range(3)]
    ws = torch.empty(fa.bwd_workspace_bytes(B, H, N, d), device="cuda", dtype=torch.uint8)
    assert lib.fa_bwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o1.data_ptr(), l1.data_ptr(), do.data_ptr(),
                          g2[0].data_ptr(), g2[1].data_ptr(), g2[2].data_ptr(), ws.data_ptr(), ws.numel(),
                          B, H, H, N, d, w.scale, 1, st) == 0
    torch.cuda.synchronize()
    i16 = torch.int16
    assert torch.equal(o1.view(i16), o2.view(i16)) and torch.equal(l1, l2)
    assert torch.equal(g1[1].view(i16), g2[1].view(i16)) and torch.equal(g1[2].view(i16), g2[2].view(i16))
    assert max_abs(host(g1[0]), host(g2[0])) <= 2e-2


def test_gqa_dk_dv_deterministic(fa):
    import torch
    w, x, (q, k, v, do) = _inputs(1700, 1, 8, 2, 700, 128, True)
    announce("fa_bwd_gqa repeat")
    o, lse = fa.fwd(q, k, v, causal=True)
    g1 = fa.bwd(q, k, v, o, lse, do, causal=True)
    g2 = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(g1[1:], g2[1:]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_gqa_long_context_sampled_heads(fa):
    """B=1, H=32 query heads over H_kv=4 K/V heads (G=8), N=4096, d=128,
    causal: one whole query head (O, LSE, dQ) and one whole K/V head (dK,
    dV, which sum its 8 query heads) against the oracle."""
    import torch
    B, H, H_kv, N, d = 1, 32, 4, 4096, 128
    w, x, (q, k, v, do) = _inputs(1800, B, H, H_kv, N, d, True)
    announce("fa_fwd_gqa/fa_bwd_gqa H=32 H_kv=4 N=4096")
    o, lse = fa.fwd(q, k, v, causal=True)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    o, lse, dq, dk, dv = (host(t) for t in (o, lse, dq, dk, dv))
    h = 13
    j = A.kv_head(h, H, H_kv)
    sl = lambda a, hh: a[:, hh:hh + 1]
    o_ref, l_ref = A.forward_gqa(sl(x["q"], h), sl(x["k"], j), sl(x["v"], j), w.scale, True)
    assert max_abs(o[:, h], o_ref[:, 0]) <= 2e-2 and max_abs(lse[:, h], l_ref[:, 0]) <= 1e-3
    G = H // H_kv
    grp = slice(j * G, (j + 1) * G)
    ref = A.backward_gqa(x["q"][:, grp], sl(x["k"], j), sl(x["v"], j), x["do"][:, grp], w.scale, True)
    _check_grads([dq[:, grp], dk[:, j:j + 1], dv[:, j:j + 1]], ref, "gqa H=32/4 N=4096 group 1")


@pytest.mark.parametrize("B,H,H_kv,N,d", [(64, 4, 2, 4096, 64), (64, 8, 1, 2048, 128)])
def test_gqa_large_batches(fa, B, H, H_kv, N, d):
    """Many batches: sampled (batch, K/V head) pairs against the oracle, and
    dK/dV bits repeatable (per-head float32 sums added in a fixed order)."""
    import torch
    assert fa.bwd_gqa_workspace_bytes(B, H, H_kv, N, d) == \
        fa.bwd_workspace_bytes(B, H, N, d) + 2 * B * H * N * d * 4
    w, x, (q, k, v, do) = _inputs(1900 + H, B, H, H_kv, N, d, True)
    announce(f"fa_bwd_gqa B={B} H={H} H_kv={H_kv} N={N} d={d}")
    o, lse = fa.fwd(q, k, v, causal=True)
    g1 = fa.bwd(q, k, v, o, lse, do, causal=True)
    g2 = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(g1[1:], g2[1:]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    dq, dk, dv = (host(t) for t in g1)
    G = H // H_kv
    for b, j in ((3, H_kv - 1), (B - 1, 0)):
        grp = slice(j * G, (j + 1) * G)
        ref = A.backward_gqa(x["q"][b:b + 1, grp], x["k"][b:b + 1, j:j + 1], x["v"][b:b + 1, j:j + 1],
                             x["do"][b:b + 1, grp], w.scale, True)
        _check_grads([dq[b:b + 1, grp], dk[b:b + 1, j:j + 1], dv[b:b + 1, j:j + 1]], ref,
                     f"gqa batch {b} K/V head {j}")

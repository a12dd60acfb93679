"""Packed variable-length batches on the GPU against the float64 oracle
(oracle.attention.forward_varlen / backward_varlen).

Inputs: seeded bf16 tensors in the packed layout [H, T, d] ([H_kv, T, d] for
K and V) with a seeded mix of lengths, including empty and one-row
sequences. Tolerances are the bf16 ones of the plain path (O within 2e-2,
LSE within 1e-3; gradients within max(2e-2, one bf16 spacing at |ref|)).
"""

import numpy as np
import pytest

import seeded_inputs as si
from gpu_util import announce, bf16_ulp, host, max_abs
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


def _packed(seed, lens, H, H_kv, d):
    """Seeded bf16 q, k, v, do in the packed layout, with their float values."""
    import torch
    T = int(sum(lens))
    rng = np.random.default_rng(seed)
    out, vals = [], {}
    for name, h in (("q", H), ("k", H_kv), ("v", H_kv), ("do", H)):
        bits, x = si.bf16_round(si.draw_normal(rng, (h, T, d)))
        vals[name] = x
        out.append(torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda())
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return vals, out, cu, torch.from_numpy(cu).cuda()


def _check_grads(got, ref, what):
    for n, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert np.all(np.isfinite(g)), f"{what} {n} not finite"
        bound = np.maximum(2e-2, bf16_ulp(r))
        assert np.all(np.abs(g - r) <= bound), f"{what} {n}: max-abs {max_abs(g, r):.3e}"


LENGTH_MIXES = {
    "ragged": [300, 1, 0, 517, 64, 255, 257],
    "one long": [1200, 3, 40],
    "equal": [256, 256, 256],
    "single": [777],
    "mostly empty": [0, 0, 5, 0, 1, 0],
}


@pytest.mark.parametrize("mix", sorted(LENGTH_MIXES))
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,H_kv", [(2, 2), (4, 2)])
def test_varlen_parity(fa, mix, d, causal, H, H_kv):
    import torch
    lens = LENGTH_MIXES[mix]
    vals, (q, k, v, do), cu, cu_t = _packed(2100 + len(lens) + d + 7 * H_kv, lens, H, H_kv, d)
    scale = 1 / np.sqrt(d)
    announce(f"fa_fwd_varlen/fa_bwd_varlen {mix} H={H} H_kv={H_kv} d={d} causal={causal}")
    o, lse = fa.fwd_varlen(q, k, v, cu_t, max(lens), causal=causal)
    dq, dk, dv = fa.bwd_varlen(q, k, v, o, lse, do, cu_t, max(lens), causal=causal)
    torch.cuda.synchronize()
    o_ref, l_ref = A.forward_varlen(vals["q"], vals["k"], vals["v"], cu, scale, causal)
    assert max_abs(host(o), o_ref) <= 2e-2
    assert max_abs(host(lse), l_ref) <= 1e-3
    ref = A.backward_varlen(vals["q"], vals["k"], vals["v"], vals["do"], cu, scale, causal)
    _check_grads([host(t) for t in (dq, dk, dv)], ref, f"varlen {mix} d={d} causal={causal} H={H}/{H_kv}")


def test_varlen_equal_lengths_match_the_batched_path(fa):
    """B sequences of one length N packed are the [B, H, N, d] problem: the
    forward and dK/dV bit for bit, dQ to its float32 atomic order."""
    import torch
    B, H, N, d = 3, 2, 700, 128
    vals, (q, k, v, do), cu, cu_t = _packed(2200, [N] * B, H, H, d)
    announce("fa_fwd_varlen vs fa_fwd")
    o, lse = fa.fwd_varlen(q, k, v, cu_t, N, causal=True)
    g = fa.bwd_varlen(q, k, v, o, lse, do, cu_t, N, causal=True)
    to_b = lambda t: t.view(t.shape[0], B, N, t.shape[-1]).transpose(0, 1).contiguous()
    qb, kb, vb, dob = (to_b(t) for t in (q, k, v, do))
    o2, lse2 = fa.fwd(qb, kb, vb, causal=True)
    g2 = fa.bwd(qb, kb, vb, o2, lse2, dob, causal=True)
    torch.cuda.synchronize()
    i16 = torch.int16
    assert torch.equal(to_b(o).view(i16), o2.view(i16))
    assert torch.equal(lse.view(H, B, N).transpose(0, 1).contiguous(), lse2)
    assert torch.equal(to_b(g[1]).view(i16), g2[1].view(i16)) and torch.equal(to_b(g[2]).view(i16), g2[2].view(i16))
    assert max_abs(host(to_b(g[0])), host(g2[0])) <= 2e-2


def test_varlen_long_mix_sampled(fa):
    """A 16-sequence mix up to 8192 rows (H=8, d=128, causal): the two
    longest and one short sequence of one head against the oracle."""
    import torch
    rng = np.random.default_rng(2300)
    lens = [int(x) for x in rng.integers(1, 8193, size=16)]
    H, d = 8, 128
    vals, (q, k, v, do), cu, cu_t = _packed(2301, lens, H, H, d)
    announce(f"fa_fwd_varlen/fa_bwd_varlen 16 sequences, T={sum(lens)}")
    o, lse = fa.fwd_varlen(q, k, v, cu_t, max(lens), causal=True)
    dq, dk, dv = fa.bwd_varlen(q, k, v, o, lse, do, cu_t, max(lens), causal=True)
    torch.cuda.synchronize()
    o, lse, dq, dk, dv = (host(t) for t in (o, lse, dq, dk, dv))
    scale = 1 / np.sqrt(d)
    order = np.argsort(lens)
    h = 5
    for b in (order[-1], order[-2], order[0]):
        r0, r1 = cu[b], cu[b + 1]
        sl = lambda x: x[h:h + 1, r0:r1]
        o_ref, l_ref = A.forward_varlen(sl(vals["q"]), sl(vals["k"]), sl(vals["v"]), [0, r1 - r0], scale, True)
        assert max_abs(o[h:h + 1, r0:r1], o_ref) <= 2e-2 and max_abs(lse[h:h + 1, r0:r1], l_ref) <= 1e-3
        ref = A.backward_varlen(sl(vals["q"]), sl(vals["k"]), sl(vals["v"]), sl(vals["do"]), [0, r1 - r0], scale, True)
        _check_grads([dq[h:h + 1, r0:r1], dk[h:h + 1, r0:r1], dv[h:h + 1, r0:r1]], ref, f"varlen seq {b} len {r1 - r0}")

"""Backward of the fp8 forward on the GPU (fa_dequant_fp8, fa_bwd_fp8).

Reading ("FlashAttention v1～v4 完整进化史" puts fp8 in the forward only): the
gradients are those of attention at the dequantised Q, K, V, formed by the
backward step of "6.1 FlashAttention V1详解" (sections 6.1-6.2) from the fp8
forward's saved O and L. References and bounds come from the oracle only:
  * decoding: bf16 values bit-exact against the oracle's decode(code) * s for
    power-of-two scales; a block with any other scale comes out NaN;
  * the backward: codes from the oracle's quantiser (power-of-two scales,
    rotated Q and K, outlier channels), O and L from the oracle's fp8
    emulation (O rounded to bf16, L to float32), dO seeded; reference
    oracle.fp8.fp8_backward on the same values; bound: the bf16 gradient bound
    of the backward tests plus the propagated bf16 rounding of P and dS
    (tests/gpu_util.grad_rounding_bound), on oracle values.
"""

import numpy as np
import pytest

import seeded_inputs as si
from gpu_util import announce, bf16_ulp, grad_rounding_bound, host, max_abs
from oracle import fp8 as F

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import exact_tiled_attention_12_amd as m
    m.load()
    return m


def _dev(a, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).cuda()


def _bf16_dev(vals):
    import torch
    bits, v = si.bf16_round(np.asarray(vals, dtype=np.float32))
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda(), v


@pytest.mark.parametrize("block_rows", [64, 0])
@pytest.mark.parametrize("N", [1, 65, 200])
def test_dequant_exact_for_power_of_two_scales(fa, N, block_rows):
    import torch
    w = si.Workload(1990 + N, "dequant", 2, 3, N, 128, "bf16", False, False, outlier_frac=0.01,
                    outlier_gain=30.0)
    x = si.make_inputs(w, names=("q",))["q"].copy()
    x[0, 0, :min(N, 3)] *= np.float32(1e-4)     # small values: subnormal codes
    codes, s, _ = F.quantize(x, block_rows, pow2=True)
    announce(f"fa_dequant_fp8 N={N} block_rows={block_rows}")
    out = fa.dequant_fp8(_dev(codes, torch.uint8), _dev(s, torch.float32), block_rows=block_rows)
    torch.cuda.synchronize()
    ref = F.dequantize(codes, s, block_rows if block_rows else 64)
    bits, ref_b = si.bf16_round(ref.astype(np.float32))
    assert np.array_equal(ref_b.astype(np.float64), ref), "power-of-two products must be exact in bf16"
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, bits)


def test_dequant_refuses_other_scales(fa):
    import torch
    N = 130
    rng = np.random.default_rng(1995)
    x = rng.standard_normal((1, 2, N, 128)).astype(np.float32)
    codes, s, _ = F.quantize(x, 64, pow2=True)
    s = s.copy()
    s[0, 1, 1] *= np.float32(1.25)
    announce("fa_dequant_fp8 non-power-of-two scale")
    out = host(fa.dequant_fp8(_dev(codes, torch.uint8), _dev(s, torch.float32)))
    assert np.all(np.isnan(out[0, 1, 64:128]))
    assert np.all(np.isfinite(out[0, 1, :64])) and np.all(np.isfinite(out[0, 1, 128:]))
    assert np.all(np.isfinite(out[0, 0]))


def _case(N, d, causal, seed):
    w = si.Workload(seed, "fp8 bwd", 1, 2, N, d, "bf16", causal, True, outlier_frac=0.01, outlier_gain=30.0,
                    rotate=True)
    x = si.make_inputs(w, names=("q", "k", "v", "do"))
    qc = F.quantize(x["q"], 64, x["rot"], pow2=True)
    kc = F.quantize(x["k"], 64, x["rot"], pow2=True)
    vc = F.quantize(x["v"], 64, pow2=True)
    codes = (qc[0], qc[1], kc[0], kc[1], vc[0], vc[1])
    o_em, l_em = F.fp8_attention_tiled(*codes, w.scale, causal)
    o_bits, o_b = si.bf16_round(o_em.astype(np.float32))
    l_f = l_em.astype(np.float32)
    return w, x, codes, o_bits, o_b.astype(np.float64), l_f


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(17, 128), (64, 128), (65, 128), (200, 128), (257, 128), (200, 64), (700, 128)])
def test_bwd_fp8_against_oracle(fa, N, d, causal):
    import torch
    w, x, codes, o_bits, o_b, l_f = _case(N, d, causal, 2000 + N + d)
    q8, sq, k8, sk, v8, sv = codes
    t8 = [_dev(c, torch.uint8) for c in (q8, k8, v8)]
    ts = [_dev(c, torch.float32) for c in (sq, sk, sv)]
    o_dev = torch.from_numpy(o_bits.view(np.int16)).view(torch.bfloat16).cuda()
    do_dev = torch.from_numpy(np.ascontiguousarray(x["do_bits"]).view(np.int16)).view(torch.bfloat16).cuda()
    announce(f"fa_bwd_fp8 N={N} d={d} causal={causal}")
    grads = fa.bwd_fp8(t8[0], t8[1], t8[2], ts[0], ts[1], ts[2], o_dev, _dev(l_f, torch.float32), do_dev,
                       causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    do = x["do"].astype(np.float64)
    ref = F.fp8_backward(*codes, o_b, l_f.astype(np.float64), do, w.scale, causal)
    qd, kd, vd = (F.dequantize(c, s, 64) for c, s in ((q8, sq), (k8, sk), (v8, sv)))
    heads = [grad_rounding_bound(qd[0, h], kd[0, h], vd[0, h], o_b[0, h], l_f[0, h].astype(np.float64),
                                 do[0, h], w.scale, causal) for h in range(2)]
    worst = []
    for name, g, r, i in zip(("dQ", "dK", "dV"), grads, ref, range(3)):
        g = host(g)
        assert np.all(np.isfinite(g)), f"{name} not finite"
        extra = np.stack([b[i] for b in heads])[None]
        bound = np.maximum(2e-2, bf16_ulp(r)) + extra
        worst.append(float(np.max(np.abs(g - r) / bound)))
        assert bool(np.all(np.abs(g - r) <= bound)), f"{name} max-abs {max_abs(g, r):.3e}"
    print(f"fp8 bwd N={N} d={d} causal={causal}: worst err/bound dQ {worst[0]:.3f} dK {worst[1]:.3f} "
          f"dV {worst[2]:.3f}")


def test_bwd_fp8_refuses_other_scales(fa):
    """A Q block whose scale is not a power of two decodes to NaN, and so do
    the gradients it reaches (its dQ rows); other heads stay finite."""
    import torch
    w, x, codes, o_bits, o_b, l_f = _case(200, 128, False, 2400)
    q8, sq, k8, sk, v8, sv = codes
    sq = sq.copy()
    sq[0, 1, 1] *= np.float32(1.5)
    o_dev = torch.from_numpy(o_bits.view(np.int16)).view(torch.bfloat16).cuda()
    do_dev = torch.from_numpy(np.ascontiguousarray(x["do_bits"]).view(np.int16)).view(torch.bfloat16).cuda()
    announce("fa_bwd_fp8 non-power-of-two Q scale")
    dq, dk, dv = fa.bwd_fp8(_dev(q8, torch.uint8), _dev(k8, torch.uint8), _dev(v8, torch.uint8),
                            _dev(sq, torch.float32), _dev(sk, torch.float32), _dev(sv, torch.float32), o_dev,
                            _dev(l_f, torch.float32), do_dev, causal=False, scale=w.scale)
    dq, dk, dv = host(dq), host(dk), host(dv)
    assert np.all(np.isnan(dq[0, 1, 64:128]))
    assert np.all(np.isfinite(dq[0, 0])) and np.all(np.isfinite(dk[0, 0])) and np.all(np.isfinite(dv[0, 0]))

"""fa_bwd_noalloc against fa_bwd, through the C ABI.

fa_bwd_noalloc is fa_bwd for callers that cannot allocate: its workspace is
a fixed array inside the library (one per device) and the (batch, head)
pairs run in chunks that fit it. Two calls in a row on the same device
share that array; the second is smaller than the first, so a stale first
call's accumulator would show. The comparison is with fa_bwd on the same
inputs: dK and dV are formed by the same per-workgroup instruction stream
and must be bit-identical; dQ is summed with float32 atomics in an order
that varies, so it must agree to the rounding of that sum (two bf16
spacings) and lie within the bf16 gradient tolerance of the backward tests.
"""

import ctypes

import numpy as np
import pytest

from gpu_util import announce, bf16_ulp, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import exact_tiled_attention_12_amd as m
    m.load()
    return m


def _inputs(B, H, N, d, causal, seed):
    import torch
    gen = torch.Generator(device="cuda").manual_seed(seed)
    mk = lambda: torch.randn((B, H, N, d), device="cuda", generator=gen, dtype=torch.float32).to(torch.bfloat16)
    return mk(), mk(), mk(), mk()


def _noalloc(fa, q, k, v, o, lse, do, causal, scale):
    import torch
    from exact_tiled_attention_12_amd import _lib
    B, H, N, d = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    stream = torch.cuda.current_stream().cuda_stream
    st = _lib.load().fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                    do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                    B, H, N, d, ctypes.c_float(scale), int(causal), stream or None)
    _lib.check(st, "fa_bwd_noalloc")
    return dq, dk, dv


# (B, H, N, d, causal): the first needs two chunks of the scratch array
# (15 heads of N = 16384, d = 128 fit it), the second is smaller.
CALLS = [(1, 20, 16384, 128, True), (2, 3, 1000, 64, False)]


def test_noalloc_matches_fa_bwd_on_two_calls(fa):
    import torch
    from exact_tiled_attention_12_amd import _lib
    lib = _lib.load()
    assert lib.fa_bwd_noalloc_scratch_bytes() == 128 << 20
    for i, (B, H, N, d, causal) in enumerate(CALLS):
        scale = 1.0 / np.sqrt(d)
        q, k, v, do = _inputs(B, H, N, d, causal, 7100 + i)
        announce(f"fa_bwd_noalloc call {i}: B={B} H={H} N={N} d={d} causal={causal}")
        o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
        got = _noalloc(fa, q, k, v, o, lse, do, causal, scale)
        ref = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(got[1].view(torch.int16), ref[1].view(torch.int16)), f"call {i}: dK differs"
        assert torch.equal(got[2].view(torch.int16), ref[2].view(torch.int16)), f"call {i}: dV differs"
        g, r = host(got[0]), host(ref[0])
        assert np.all(np.isfinite(g)), f"call {i}: dQ not finite"
        assert np.all(np.abs(g - r) <= 2 * bf16_ulp(r) + 1e-6), f"call {i}: dQ max diff {np.max(np.abs(g - r)):.3e}"
        assert np.all(np.abs(g - r) <= np.maximum(2e-2, bf16_ulp(r))), f"call {i}: dQ beyond the bf16 tolerance"
        del q, k, v, do, o, lse, got, ref

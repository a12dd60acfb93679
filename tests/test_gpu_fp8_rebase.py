"""fp8 forward on inputs that move the row reference late in the key sweep.

The fp8 forward keeps each row's reference on whole powers of two (its
running maximum rounded up: the lazy rescaling of "FlashAttention v1～v4
完整进化史", v4 part 3, read for fp8) and multiplies its float32 accumulator
only when that reference passes the accumulator's own by more than 2^8
(log2 units). Random N(0, 1) inputs settle the maximum in the first tile, so
these cases make it move later:
  * growing keys: key row j scaled by 1 + 5 j / N, so the maxima of late
    tiles exceed those of early ones by far more than 8 (log2 units);
  * a spike: one key row scaled by 24;
  * shrinking keys: the first tiles hold the largest keys (fewer late moves).
The growing and spike cases first check, on the oracle's dequantised scores
(CPU), that the inputs do what they are meant to (some rows' reference passes
the accumulator's by more than 2^8 after the row's first key); every case
then compares the GPU result with the oracle's fp8 emulation on the same
codes within tests/fp8_bounds.py's element bound.
"""

import numpy as np
import pytest

from fp8_bounds import bound_rows
from gpu_util import announce
from oracle import fp8 as F

pytestmark = pytest.mark.gpu

D = 128
BC = 64          # keys per tile of the kernel and the emulation
THRESH = 8.0     # log2 units the reference may run ahead of the accumulator's


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import exact_tiled_attention_12_amd as m
    m.load()
    return m


def _codes(kind: str, N: int, seed: int):
    rng = np.random.default_rng(seed)
    x = {n: rng.standard_normal(size=(1, 2, N, D), dtype=np.float32) for n in "qkv"}
    j = np.arange(N, dtype=np.float32)
    if kind == "growing":
        x["k"] *= (1.0 + 5.0 * j / N)[None, None, :, None]
    elif kind == "shrinking":
        x["k"] *= (6.0 - 5.0 * j / N)[None, None, :, None]
    elif kind == "spike":
        x["k"][:, :, min(300, N - 1)] *= 24.0
    else:
        raise ValueError(kind)
    q8, sq, _ = F.quantize(x["q"], 64)
    k8, sk, _ = F.quantize(x["k"], 64)
    v8, sv, _ = F.quantize(x["v"], 64, pow2=True)
    return q8, sq, k8, sk, v8, sv


def _late_rebases(codes, h, scale, causal):
    """Rows of head h whose power-of-two reference passes the accumulator's
    by more than 2^8 after the row's first key (re-bases beyond the first)."""
    q8, sq, k8, sk = codes[:4]
    qd = F.dequantize(q8, sq)[0, h]
    kd = F.dequantize(k8, sk)[0, h]
    N = qd.shape[0]
    s = scale * (qd @ kd.T) / np.log(2.0)
    if causal:
        s = np.where(np.arange(N)[None, :] > np.arange(N)[:, None], -np.inf, s)
    count = np.zeros(N, dtype=int)
    for r in range(N):
        m = mr = -np.inf
        for t0 in range(0, N, BC):
            tmax = s[r, t0:t0 + BC].max()
            if np.isfinite(tmax):
                m = max(m, np.ceil(tmax))
            if np.isfinite(m) and np.isfinite(mr) and m - mr > THRESH:
                count[r] += 1
            if np.isfinite(m) and not np.isfinite(mr):
                mr = m
            elif m - mr > THRESH:
                mr = m
    return count


CASES = [(kind, N, causal) for kind in ("growing", "spike", "shrinking") for N in (700, 1500)
         for causal in (False, True)]


@pytest.mark.parametrize("kind,N,causal", CASES)
def test_fwd_fp8_late_maximum(fa, kind, N, causal):
    import torch
    codes = _codes(kind, N, 2600 + N)
    scale = 1.0 / np.sqrt(D)
    late = [_late_rebases(codes, h, scale, causal) for h in range(2)]
    n_late = int(sum(int(np.count_nonzero(c)) for c in late))
    if kind != "shrinking":
        assert n_late > 0, f"{kind} inputs must move the reference past the accumulator's"
    t = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in codes]
    announce(f"fa_fwd_fp8 late maximum {kind} N={N} causal={causal} ({n_late} rows re-based late)")
    o, lse = fa.fwd_fp8(t[0], t[2], t[4], t[1], t[3], t[5], causal=causal, scale=scale)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    q8, sq, k8, sk, v8, sv = codes
    worst_o = worst_l = 0.0
    for h in range(2):
        rows = np.arange(N)
        ob, lb, o_em, l_em = bound_rows(q8[0, h], sq[0, h], k8[0, h], sk[0, h], v8[0, h], sv[0, h], scale,
                                        causal, rows)
        assert np.all(np.isfinite(o[0, h])) and np.all(np.isfinite(lse[0, h]))
        worst_o = max(worst_o, float(np.max(np.abs(o[0, h] - o_em) / ob)))
        worst_l = max(worst_l, float(np.max(np.abs(lse[0, h] - l_em) / lb)))
    print(f"fp8 late maximum {kind} N={N} causal={causal}: {n_late} rows re-based late, "
          f"O err/bound {worst_o:.3f}, LSE err/bound {worst_l:.3f}")
    assert worst_o <= 1.0 and worst_l <= 1.0, (worst_o, worst_l)

"""Scale-granularity study of the fp8 path, on the oracle alone (CPU).

Test infrastructure: this script imports only ``oracle`` and the seeded input
generators, never the GPU library.

"FlashAttention v1～v4 完整进化史", v3 part 3 (FP8): per-block scales and an
orthogonal rotation of Q and K keep outlier channels from spending the fp8
range of a whole tensor. This script measures how the attention error of the
fp8 path depends on the choices the page leaves open, on the 4 x 32 x 8192 x
128 fp8 workload (four shared outlier channels x30 in Q, K and V; one Haar
rotation), over eight heads (the outlier heads, then seeded random ones):

  * rows per scale block: 64, 128, 256, 1024, or one scale per tensor;
  * rotation of Q and K on or off;
  * the form of a scale: the smallest power of two at or above amax/448,
    amax/448 itself, or amax/448 for Q and K with a power of two for V.

Every variant runs the oracle's tiled fp8 attention (P rounded through e4m3
as the kernel does) against the exact float64 attention of the unquantised
inputs, and prints the RMSE of O. Usage:

    python oracle/fp8_granularity.py [--heads 8] [--procs 8] [--blocks 64,0] [--forms pow2,exact,mixed]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from oracle import attention as A  # noqa: E402
from oracle import fp8 as F  # noqa: E402
import seeded_inputs as si  # noqa: E402

BLOCKS = (64, 128, 256, 1024, 0)
REFERENCE = os.environ.get("FP8_REFERENCE", "pow2")   # the emulation's row reference (see fp8_attention_tiled)


def sample_heads(x, w, n):
    heads = sorted({(0, int(h)) for h in x["outliers"][:, 0]})
    rng = np.random.default_rng(5)
    while len(heads) < n:
        bh = (int(rng.integers(w.B)), int(rng.integers(w.H)))
        if bh not in heads:
            heads.append(bh)
    return heads[:n]


def head_scales(xf, block_rows, pow2, amax_tensor):
    """Scales of one head [1, 1, N, d]; per tensor, from the whole tensor's amax."""
    if block_rows == 0:
        one = np.full((1, 1, 1, 1), amax_tensor, dtype=np.float32)
        s = F.block_scales(one, 0, pow2)[0, 0, 0]
        return np.full((1, 1, -(-xf.shape[2] // 64)), s, dtype=np.float32)
    return F.block_scales(xf, block_rows, pow2)


def quant_head(x, block_rows, rot, form, amax_tensor):
    """Codes and scales of one head [1, 1, N, d] (rotation taken in float64)."""
    x = np.asarray(x, dtype=np.float64)
    if rot is not None:
        x = x @ np.asarray(rot, dtype=np.float64)
    xf = x.astype(np.float32)
    s = head_scales(xf, block_rows, form == "pow2", amax_tensor)
    br = block_rows if block_rows > 0 else 64
    srow = s[:, :, np.arange(xf.shape[2]) // br][..., None]
    return F.e4m3_encode((xf / srow).astype(np.float32)), s


def tensor_amax(x):
    """amax of Q, K (with and without the rotation) and V over the whole tensor."""
    out = {}
    for n in ("q", "k", "v"):
        out[n] = {False: float(np.max(np.abs(x[n])))}
        if n != "v":
            out[n][True] = max(float(np.max(np.abs(np.asarray(x[n][b], np.float64) @ x["rot"])))
                               for b in range(x[n].shape[0]))
    return out


def one_head(args):
    (b, h), variants, amax = args
    w = si.workload(5)
    x = si.make_inputs(w, names=("q", "k", "v"))
    q, k, v = (x[n][b:b + 1, h:h + 1] for n in ("q", "k", "v"))
    o_ex, _ = A.forward(q[0, 0], k[0, 0], v[0, 0], w.scale, False)
    out = {}
    for br, rot, form in variants:
        R = x["rot"] if rot else None
        qk_form = "exact" if form == "mixed" else form
        v_form = "pow2" if form == "mixed" else form
        q8, sq = quant_head(q, br, R, qk_form, amax["q"][rot])
        k8, sk = quant_head(k, br, R, qk_form, amax["k"][rot])
        v8, sv = quant_head(v, br, None, v_form, amax["v"][False])
        o, _ = F.fp8_attention_tiled(q8, sq, k8, sk, v8, sv, w.scale, False, block_rows=br if br else 64,
                                     reference=REFERENCE)
        out[(br, rot, form)] = float(np.sum((o[0, 0] - o_ex) ** 2)), o_ex.size
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--heads", type=int, default=8)
    ap.add_argument("--procs", type=int, default=8)
    ap.add_argument("--blocks", default=",".join(str(b) for b in BLOCKS), help="rows per block; 0 = per tensor")
    ap.add_argument("--forms", default="pow2,exact,mixed",
                    help="scale forms: pow2, exact, mixed (Q and K exact, V a power of two)")
    args = ap.parse_args()
    os.environ["OPENBLAS_NUM_THREADS"] = "1"   # inherited by the workers
    w = si.workload(5)
    x = si.make_inputs(w, names=("q", "k", "v"))
    heads = sample_heads(x, w, args.heads)
    amax = tensor_amax(x)
    del x
    forms = args.forms.split(",")
    blocks = [int(b) for b in args.blocks.split(",")]
    variants = [(br, rot, form) for br in blocks for rot in (True, False) for form in forms]
    t0 = time.time()
    import multiprocessing as mp
    with mp.get_context("spawn").Pool(min(args.procs, len(heads))) as pool:
        res = pool.map(one_head, [(bh, variants, amax) for bh in heads])
    se = {v: sum(r[v][0] for r in res) for v in variants}
    n = sum(res[0][variants[0]][1] for _ in res)
    table = {f"{'tensor' if br == 0 else br}|{'rot' if rot else 'norot'}|{form}": float(np.sqrt(se[(br, rot, form)] / n))
             for br, rot, form in variants}
    print(json.dumps({"heads": heads, "seconds": round(time.time() - t0, 1), "rmse": table}, indent=1))


if __name__ == "__main__":
    main()

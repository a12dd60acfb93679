"""Seeded synthetic inputs for the attention workloads.

This module is shared by the float64 oracle's tests, the GPU parity tests and
the benchmark. It holds no attention arithmetic: only random draws, the
round-to-nearest-even cast of those draws to bf16 (the dtype the workloads are
stated in), the choice of outlier channels, and the random orthogonal matrix
that the fp8 path consumes as an input.

Workloads (one GPU each; shapes are [B, H, N, d], row-major, contiguous):

  1  B=1  H=1  N=256   d=64   fp32  no mask  forward only
  2  B=8  H=12 N=1024  d=64   bf16  no mask  forward only
  3  B=2  H=32 N=4096  d=128  bf16  causal   forward only
  4  B=1  H=32 N=16384 d=128  bf16  causal   forward + backward
  5  B=4  H=32 N=8192  d=128  fp8   no mask  forward, outliers + rotation

Recipe: workload k draws from ``np.random.default_rng(1000 + k)``; the
standard normals are drawn as float32 in the order Q, K, V, dO and then rounded
to the workload dtype with round-to-nearest-even.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "bf16_round", "bf16_bits_to_f32",
    "draw_normal", "make_inputs", "outlier_channels", "haar_orthogonal",
]


@dataclass(frozen=True)
class Workload:
    id: int
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "f32", "bf16" or "fp8"
    causal: bool
    backward: bool
    outlier_frac: float = 0.0
    outlier_gain: float = 1.0
    rotate: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def seed(self) -> int:
        return 1000 + self.id

    def resized(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    1: Workload(1, "single-head fp32 d64 N256", 1, 1, 256, 64, "f32", False, False),
    2: Workload(2, "non-causal bf16 d64 N1024 B8 H12", 8, 12, 1024, 64, "bf16", False, False),
    3: Workload(3, "causal bf16 d128 N4096 B2 H32", 2, 32, 4096, 128, "bf16", True, False),
    4: Workload(4, "causal bf16 d128 N16384 B1 H32 fwd+bwd", 1, 32, 16384, 128, "bf16", True, True),
    5: Workload(5, "fp8 e4m3 d128 N8192 B4 H32 non-causal", 4, 32, 8192, 128, "fp8", False, False,
                outlier_frac=0.001, outlier_gain=30.0, rotate=True),
}


def workload(k: int) -> Workload:
    return WORKLOADS[k]


def bf16_round(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Round float32 values to bf16 with round-to-nearest-even.

    Returns (bits as uint16, the rounded values as float32). NaN stays NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint32)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, (u >> 16).astype(np.uint32) | 0x40, r)
    bits = r.astype(np.uint16)
    vals = (bits.astype(np.uint32) << 16).view(np.float32)
    return bits, vals


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def draw_normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def outlier_channels(rng: np.random.Generator, H: int, d: int, frac: float) -> np.ndarray:
    """Pick round(frac * H * d) (at least 1) distinct (head, dim) channels.

    Returns an int array of shape [n, 2] holding (head, dim) pairs.
    """
    n = max(1, int(round(frac * H * d)))
    flat = rng.choice(H * d, size=n, replace=False)
    return np.stack([flat // d, flat % d], axis=1).astype(np.int64)


def haar_orthogonal(rng: np.random.Generator, d: int) -> np.ndarray:
    """Draw a d x d orthogonal matrix from the Haar measure.

    QR of a float64 Gaussian matrix with the columns of Q multiplied by the
    signs of diag(R) (without that fix the draw is not uniform). Returns
    float64; callers store it as float32.
    """
    g = rng.standard_normal(size=(d, d))
    qm, r = np.linalg.qr(g)
    s = np.sign(np.diag(r))
    s[s == 0] = 1.0
    return qm * s[None, :]


def make_inputs(w: Workload, names=("q", "k", "v", "do")) -> dict:
    """Draw the tensors of workload ``w``.

    Returns a dict name -> float32 array holding the values in the workload's
    storage precision (bf16-rounded for bf16 and fp8 workloads), plus
    ``name + "_bits"`` (uint16) for bf16-stored tensors. For the fp8 workload
    the dict also holds ``rot`` (float32 d x d orthogonal matrix) and
    ``outliers`` (the (head, dim) pairs scaled by the outlier gain in Q, K
    and V). The fp8 workload's Q, K, V are stored in bf16 before quantisation.
    """
    rng = np.random.default_rng(w.seed)
    shape = (w.B, w.H, w.N, w.d)
    out = {}
    raw = {}
    for nm in ("q", "k", "v", "do"):
        # Always draw in the fixed order so that a subset of names does not
        # change the values of the others.
        x = draw_normal(rng, shape)
        if nm in names:
            raw[nm] = x
        else:
            del x
    if w.outlier_frac > 0:
        ch = outlier_channels(rng, w.H, w.d, w.outlier_frac)
        out["outliers"] = ch
        for nm in ("q", "k", "v"):
            if nm in raw:
                for hh, dd in ch:
                    raw[nm][:, hh, :, dd] *= np.float32(w.outlier_gain)
    if w.rotate:
        out["rot"] = haar_orthogonal(rng, w.d).astype(np.float32)
    for nm, x in raw.items():
        if w.dtype == "f32":
            out[nm] = x
        else:
            bits, vals = bf16_round(x)
            out[nm] = vals
            out[nm + "_bits"] = bits
    return out

"""Python binding over the C ABI: argument marshalling only.

torch supplies device memory and the current HIP stream; every step of the
computation runs in the library's kernels. Shapes are [B, H, N, d].
"""

from __future__ import annotations

import math

import torch

from . import _lib

__all__ = ["fwd", "bwd", "bwd_stages", "bwd_workspace_bytes", "bwd_det_workspace_bytes", "bwd_gqa_workspace_bytes",
           "fwd_varlen", "bwd_varlen", "quant_fp8", "fwd_fp8", "dequant_fp8", "bwd_fp8", "bwd_fp8_workspace_bytes"]


def _stream(t: torch.Tensor):
    return ctypes_ptr(torch.cuda.current_stream(t.device).cuda_stream)


def ctypes_ptr(x: int):
    return x if x else None


def _check_tensor(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _shape4(q: torch.Tensor):
    if q.dim() != 4:
        raise ValueError(f"expected a [B, H, N, d] tensor, got shape {tuple(q.shape)}")
    return tuple(int(x) for x in q.shape)


def _kv_heads(q, k):
    """K/V heads of k ([B, H_kv, N, d]); H_kv < H selects grouped-query attention (bf16)."""
    B, H, N, d = _shape4(q)
    H_kv = int(k.shape[1]) if k.dim() == 4 else -1
    if H_kv != H and (H_kv < 1 or H % H_kv or q.dtype != torch.bfloat16):
        raise ValueError(f"k has {H_kv} heads: grouped-query attention needs bf16 and H = {H} a multiple of it")
    return H_kv


def fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None):
    """O, LSE = attention(q, k, v). bf16 or float32 inputs; O has the input dtype.

    k and v may have fewer heads than q (bf16): query head h then attends with
    K/V head h // (H // H_kv) (grouped-query; one K/V head is multi-query).
    """
    B, H, N, d = _shape4(q)
    dt = q.dtype
    if dt not in (torch.bfloat16, torch.float32):
        raise TypeError(f"q must be bfloat16 or float32 (got {dt})")
    H_kv = _kv_heads(q, k)
    _check_tensor(q, "q", dt, (B, H, N, d))
    for t, n in ((k, "k"), (v, "v")):
        _check_tensor(t, n, dt, (B, H_kv, N, d))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
    _check_tensor(out, "out", dt, (B, H, N, d))
    _check_tensor(lse, "lse", torch.float32, (B, H, N))
    lib = _lib.load()
    if H_kv != H:
        st = lib.fa_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            B, H, H_kv, N, d, float(scale), int(bool(causal)), _stream(q))
        _lib.check(st, "fa_fwd_gqa")
        return out, lse
    fn = lib.fa_fwd if dt == torch.bfloat16 else lib.fa_fwd_f32
    st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
            B, H, N, d, float(scale), int(bool(causal)), _stream(q))
    _lib.check(st, "fa_fwd" if dt == torch.bfloat16 else "fa_fwd_f32")
    return out, lse


def _check_cu(cu_seqlens, device):
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise TypeError("cu_seqlens must be a 1-D int32 tensor of cumulative sequence lengths")
    if cu_seqlens.device != device or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be contiguous on the tensors' device")
    return int(cu_seqlens.numel()) - 1


def fwd_varlen(q, k, v, cu_seqlens, max_seqlen: int, causal: bool = False, scale: float | None = None,
               out=None, lse=None):
    """Packed variable-length attention: q [H, T, d], k, v [H_kv, T, d] (bf16);
    sequence b is rows cu_seqlens[b] .. cu_seqlens[b+1]-1. Returns O [H, T, d]
    and LSE [H, T]."""
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("fwd_varlen takes [H, T, d] tensors")
    H, T, d = (int(x) for x in q.shape)
    H_kv = int(k.shape[0])
    n_seq = _check_cu(cu_seqlens, q.device)
    _check_tensor(q, "q", torch.bfloat16, (H, T, d))
    for t, n in ((k, "k"), (v, "v")):
        _check_tensor(t, n, torch.bfloat16, (H_kv, T, d))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((H, T), device=q.device, dtype=torch.float32) if lse is None else lse
    _check_tensor(out, "out", torch.bfloat16, (H, T, d))
    _check_tensor(lse, "lse", torch.float32, (H, T))
    st = _lib.load().fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                   cu_seqlens.data_ptr(), n_seq, int(max_seqlen), T, H, H_kv, d, float(scale),
                                   int(bool(causal)), _stream(q))
    _lib.check(st, "fa_fwd_varlen")
    return out, lse


def bwd_varlen(q, k, v, o, lse, do, cu_seqlens, max_seqlen: int, causal: bool = False,
               scale: float | None = None, workspace=None, dq=None, dk=None, dv=None):
    """Gradients of fwd_varlen: dQ [H, T, d], dK, dV [H_kv, T, d] (bf16)."""
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("bwd_varlen takes [H, T, d] tensors")
    H, T, d = (int(x) for x in q.shape)
    H_kv = int(k.shape[0])
    n_seq = _check_cu(cu_seqlens, q.device)
    for t, n in ((q, "q"), (o, "o"), (do, "do")):
        _check_tensor(t, n, torch.bfloat16, (H, T, d))
    for t, n in ((k, "k"), (v, "v")):
        _check_tensor(t, n, torch.bfloat16, (H_kv, T, d))
    _check_tensor(lse, "lse", torch.float32, (H, T))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lib = _lib.load()
    if workspace is None:
        workspace = torch.empty(int(lib.fa_bwd_varlen_workspace_bytes(T, H, H_kv, d)), device=q.device,
                                dtype=torch.uint8)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_tensor(dq, "dq", torch.bfloat16, (H, T, d))
    for t, n in ((dk, "dk"), (dv, "dv")):
        _check_tensor(t, n, torch.bfloat16, (H_kv, T, d))
    st = lib.fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                           dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                           workspace.numel() * workspace.element_size(), cu_seqlens.data_ptr(), n_seq,
                           int(max_seqlen), T, H, H_kv, d, float(scale), int(bool(causal)), _stream(q))
    _lib.check(st, "fa_bwd_varlen")
    return dq, dk, dv


def bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(_lib.load().fa_bwd_workspace_bytes(B, H, N, d))


def bwd_gqa_workspace_bytes(B: int, H: int, H_kv: int, N: int, d: int) -> int:
    return int(_lib.load().fa_bwd_gqa_workspace_bytes(B, H, H_kv, N, d))


def bwd_det_workspace_bytes(B: int, H: int, N: int, d: int, causal: bool) -> int:
    return int(_lib.load().fa_bwd_det_workspace_bytes(B, H, N, d, int(bool(causal))))


def bwd(q, k, v, o, lse, do, causal: bool = False, scale: float | None = None,
        workspace=None, dq=None, dk=None, dv=None, deterministic: bool = False):
    """dQ, dK, dV of sum(O * dO), recomputing P from LSE. bf16 or float32.

    deterministic=True (bf16 only) calls fa_bwd_det: dQ is reduced over key
    tiles in a fixed order (counter-ordered adds, O(N) workspace), so every
    output is bit-identical from run to run.
    k and v may have fewer heads than q (bf16, fa_bwd_gqa); dk and dv then
    have k's shape and sum over each K/V head's query heads.
    """
    B, H, N, d = _shape4(q)
    dt = q.dtype
    H_kv = _kv_heads(q, k)
    if H_kv != H:
        if deterministic:
            raise ValueError("the fixed-order backward takes one K/V head per query head")
        for t, n in ((q, "q"), (o, "o"), (do, "do")):
            _check_tensor(t, n, dt, (B, H, N, d))
        for t, n in ((k, "k"), (v, "v")):
            _check_tensor(t, n, dt, (B, H_kv, N, d))
        _check_tensor(lse, "lse", torch.float32, (B, H, N))
        if scale is None:
            scale = 1.0 / math.sqrt(d)
        if workspace is None:
            workspace = torch.empty(bwd_gqa_workspace_bytes(B, H, H_kv, N, d), device=q.device, dtype=torch.uint8)
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(k) if dk is None else dk
        dv = torch.empty_like(v) if dv is None else dv
        _check_tensor(dq, "dq", dt, (B, H, N, d))
        for t, n in ((dk, "dk"), (dv, "dv")):
            _check_tensor(t, n, dt, (B, H_kv, N, d))
        st = _lib.load().fa_bwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                    do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                    workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                    B, H, H_kv, N, d, float(scale), int(bool(causal)), _stream(q))
        _lib.check(st, "fa_bwd_gqa")
        return dq, dk, dv
    if deterministic:
        if dt != torch.bfloat16:
            raise ValueError("the fixed-order backward takes bf16 tensors")
        for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
            _check_tensor(t, n, dt, (B, H, N, d))
        _check_tensor(lse, "lse", torch.float32, (B, H, N))
        if scale is None:
            scale = 1.0 / math.sqrt(d)
        if workspace is None:
            workspace = torch.empty(bwd_det_workspace_bytes(B, H, N, d, causal), device=q.device, dtype=torch.uint8)
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(q) if dk is None else dk
        dv = torch.empty_like(q) if dv is None else dv
        for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
            _check_tensor(t, n, dt, (B, H, N, d))
        st = _lib.load().fa_bwd_det(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                    do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                    workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                    B, H, N, d, float(scale), int(bool(causal)), _stream(q))
        _lib.check(st, "fa_bwd_det")
        return dq, dk, dv
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _check_tensor(t, n, dt, (B, H, N, d))
    _check_tensor(lse, "lse", torch.float32, (B, H, N))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check_tensor(t, n, dt, (B, H, N, d))
    lib = _lib.load()
    fn = lib.fa_bwd if dt == torch.bfloat16 else lib.fa_bwd_f32
    st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(),
            B, H, N, d, float(scale), int(bool(causal)), _stream(q))
    _lib.check(st, "fa_bwd" if dt == torch.bfloat16 else "fa_bwd_f32")
    return dq, dk, dv


def bwd_stages(q, k, v, o, lse, do, workspace, dq, dk, dv, stage_mask: int, causal: bool = False,
               scale: float | None = None):
    """Run selected stages of the bf16 backward (1 preprocess, 2 main, 4 finish) into given buffers."""
    B, H, N, d = _shape4(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check_tensor(t, n, torch.bfloat16, (B, H, N, d))
    _check_tensor(lse, "lse", torch.float32, (B, H, N))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = _lib.load().fa_bwd_stages(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                   do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                   workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                   B, H, N, d, float(scale), int(bool(causal)), int(stage_mask), _stream(q))
    _lib.check(st, "fa_bwd_stages")


def quant_fp8(x, rot=None, block_rows: int = 64, x8=None, scales=None, pow2: bool = False):
    """e4m3 codes (uint8) and per-64-row float32 scales of x (bf16 [B,H,N,d]).

    Scales are amax / 448, or with pow2 the smallest power of two at or above
    it (the form fwd_fp8 requires for V)."""
    B, H, N, d = _shape4(x)
    _check_tensor(x, "x", torch.bfloat16, (B, H, N, d))
    if rot is not None:
        _check_tensor(rot, "rot", torch.float32, (d, d))
    x8 = torch.empty((B, H, N, d), device=x.device, dtype=torch.uint8) if x8 is None else x8
    nb = (N + 63) // 64
    scales = torch.empty((B, H, nb), device=x.device, dtype=torch.float32) if scales is None else scales
    _check_tensor(x8, "x8", torch.uint8, (B, H, N, d))
    _check_tensor(scales, "scales", torch.float32, (B, H, nb))
    st = _lib.load().fa_quant_fp8(x.data_ptr(), rot.data_ptr() if rot is not None else None,
                                  x8.data_ptr(), scales.data_ptr(), B, H, N, d, int(block_rows), int(bool(pow2)),
                                  _stream(x))
    _lib.check(st, "fa_quant_fp8")
    return x8, scales


def fwd_fp8(q8, k8, v8, sq, sk, sv, causal: bool = False, scale: float | None = None, out=None, lse=None,
            block_rows: int = 64):
    """O (bf16), LSE from e4m3 codes with per-64-row scales (block_rows = 64)
    or one per-tensor scale broadcast in the same layout (block_rows = 0).
    sv must hold powers of two (quant_fp8(v, pow2=True)); a 256-row query
    tile whose keys meet any other V scale comes out NaN."""
    B, H, N, d = _shape4(q8)
    nb = (N + 63) // 64
    for t, n in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        _check_tensor(t, n, torch.uint8, (B, H, N, d))
    for t, n in ((sq, "sq"), (sk, "sk"), (sv, "sv")):
        _check_tensor(t, n, torch.float32, (B, H, nb))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty((B, H, N, d), device=q8.device, dtype=torch.bfloat16) if out is None else out
    lse = torch.empty((B, H, N), device=q8.device, dtype=torch.float32) if lse is None else lse
    _check_tensor(out, "out", torch.bfloat16, (B, H, N, d))
    _check_tensor(lse, "lse", torch.float32, (B, H, N))
    st = _lib.load().fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), sq.data_ptr(), sk.data_ptr(),
                                sv.data_ptr(), int(block_rows), out.data_ptr(), lse.data_ptr(), B, H, N, d, float(scale),
                                int(bool(causal)), _stream(q8))
    _lib.check(st, "fa_fwd_fp8")
    return out, lse


def dequant_fp8(x8, scales, block_rows: int = 64, out=None):
    """bf16 values decode(x8) * s (exact for power-of-two scales; NaN blocks
    where a scale is not a power of two)."""
    B, H, N, d = _shape4(x8)
    _check_tensor(x8, "x8", torch.uint8, (B, H, N, d))
    _check_tensor(scales, "scales", torch.float32, (B, H, (N + 63) // 64))
    out = torch.empty((B, H, N, d), device=x8.device, dtype=torch.bfloat16) if out is None else out
    _check_tensor(out, "out", torch.bfloat16, (B, H, N, d))
    st = _lib.load().fa_dequant_fp8(x8.data_ptr(), scales.data_ptr(), int(block_rows), out.data_ptr(),
                                    B, H, N, d, _stream(x8))
    _lib.check(st, "fa_dequant_fp8")
    return out


def bwd_fp8_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(_lib.load().fa_bwd_fp8_workspace_bytes(B, H, N, d))


def bwd_fp8(q8, k8, v8, sq, sk, sv, o, lse, do, causal: bool = False, scale: float | None = None,
            block_rows: int = 64, workspace=None, dq=None, dk=None, dv=None):
    """dQ, dK, dV (bf16) with respect to the dequantised inputs of fwd_fp8,
    from its o and lse; all three tensors quantised with pow2=True."""
    B, H, N, d = _shape4(q8)
    nb = (N + 63) // 64
    for t, n in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        _check_tensor(t, n, torch.uint8, (B, H, N, d))
    for t, n in ((sq, "sq"), (sk, "sk"), (sv, "sv")):
        _check_tensor(t, n, torch.float32, (B, H, nb))
    for t, n in ((o, "o"), (do, "do")):
        _check_tensor(t, n, torch.bfloat16, (B, H, N, d))
    _check_tensor(lse, "lse", torch.float32, (B, H, N))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = torch.empty(bwd_fp8_workspace_bytes(B, H, N, d), device=q8.device, dtype=torch.uint8)
    dq = torch.empty_like(o) if dq is None else dq
    dk = torch.empty_like(o) if dk is None else dk
    dv = torch.empty_like(o) if dv is None else dv
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check_tensor(t, n, torch.bfloat16, (B, H, N, d))
    st = _lib.load().fa_bwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), sq.data_ptr(), sk.data_ptr(),
                                sv.data_ptr(), int(block_rows), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                                workspace.numel() * workspace.element_size(), B, H, N, d, float(scale),
                                int(bool(causal)), _stream(q8))
    _lib.check(st, "fa_bwd_fp8")
    return dq, dk, dv

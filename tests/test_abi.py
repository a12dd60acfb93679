"""The C ABI on the CPU: the library loads, exports every declared call, and
rejects bad arguments before anything reaches the GPU.

Every call here fails validation, so no kernel is launched and no GPU is needed.
"""

import ctypes
import math
import os
import re

import pytest

from exact_tiled_attention_12_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

A = 0x100000          # fake, 256-byte aligned device addresses (never dereferenced)
GAP = 1 << 32


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:FA_API\s+)?(?:const\s+)?[a-z_]+\s*\*?\s*(fa_[a-z0-9_]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libfa_mi355x.so is not built; run python -m exact_tiled_attention_12_amd.build")
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert len(names) == 23, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(_lib.FAError):
        _lib.load(str(tmp_path / "nope.so"))


def _fwd(lib, q=A, k=A + GAP, v=A + 2 * GAP, o=A + 3 * GAP, lse=A + 4 * GAP,
         B=1, H=1, N=16, d=64, scale=0.125, causal=0, f32=False):
    fn = lib.fa_fwd_f32 if f32 else lib.fa_fwd
    return fn(q, k, v, o, lse, B, H, N, d, scale, causal, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), _lib.FA_ERR_INVALID),
    (dict(H=-1), _lib.FA_ERR_INVALID),
    (dict(N=0), _lib.FA_ERR_INVALID),
    (dict(d=96), _lib.FA_ERR_UNSUPPORTED),
    (dict(d=256), _lib.FA_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), _lib.FA_ERR_UNSUPPORTED),
    (dict(scale=float("inf")), _lib.FA_ERR_UNSUPPORTED),
    (dict(scale=-0.5), _lib.FA_ERR_UNSUPPORTED),
    (dict(q=None), _lib.FA_ERR_INVALID),
    (dict(lse=None), _lib.FA_ERR_INVALID),
    (dict(q=A + 8), _lib.FA_ERR_UNSUPPORTED),
    (dict(lse=A + 4 * GAP + 2), _lib.FA_ERR_UNSUPPORTED),
    (dict(o=A + 256), _lib.FA_ERR_INVALID),                 # o overlaps q
    (dict(lse=A + 3 * GAP + 64), _lib.FA_ERR_INVALID),      # lse inside o
    (dict(B=1 << 16, H=1 << 12, N=1 << 12), _lib.FA_ERR_UNSUPPORTED),
])
@pytest.mark.parametrize("f32", [False, True])
def test_forward_rejects(lib, kw, status, f32):
    assert _fwd(lib, f32=f32, **kw) == status
    msg = lib.fa_last_error().decode()
    assert msg, "a failed call must leave a reason"


def test_error_text_names_the_argument(lib):
    assert _fwd(lib, d=80) == _lib.FA_ERR_UNSUPPORTED
    assert "80" in lib.fa_last_error().decode()
    assert _fwd(lib, q=None) == _lib.FA_ERR_INVALID
    assert "q" in lib.fa_last_error().decode()
    for st in (0, -1, -2, -3, 7):
        assert lib.fa_status_string(st)


def test_workspace_is_linear_in_n(lib):
    def ws(B, H, N, d):
        return lib.fa_bwd_workspace_bytes(B, H, N, d)
    def al(x):
        return (x + 255) // 256 * 256
    for (B, H, N, d) in [(1, 1, 1, 64), (2, 3, 1000, 128), (1, 32, 16384, 128)]:
        assert ws(B, H, N, d) == al(4 * B * H * N * d) + al(4 * B * H * N)
    assert ws(1, 32, 16384, 128) < 300 * 2 ** 20     # far below one N x N fp32 matrix (1 GiB)
    assert ws(0, 1, 1, 64) == 0 and ws(1, 1, 1, 100) == 0


def _bwd(lib, ws=A + 10 * GAP, ws_bytes=None, B=1, H=1, N=16, d=64, scale=0.125, **over):
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_bytes(B, H, N, d)
    p = dict(q=A, k=A + GAP, v=A + 2 * GAP, o=A + 3 * GAP, lse=A + 4 * GAP, do=A + 5 * GAP,
             dq=A + 6 * GAP, dk=A + 7 * GAP, dv=A + 8 * GAP)
    p.update(over)
    return lib.fa_bwd(p["q"], p["k"], p["v"], p["o"], p["lse"], p["do"], p["dq"], p["dk"], p["dv"],
                      ws, ws_bytes, B, H, N, d, scale, 1, None)


def test_backward_rejects(lib):
    assert _bwd(lib, ws=None) == _lib.FA_ERR_INVALID
    assert _bwd(lib, ws_bytes=100) == _lib.FA_ERR_INVALID
    assert _bwd(lib, ws=A + 10 * GAP + 16) == _lib.FA_ERR_UNSUPPORTED
    assert _bwd(lib, dq=A + 64) == _lib.FA_ERR_INVALID           # dq overlaps q
    assert _bwd(lib, dk=A + 6 * GAP) == _lib.FA_ERR_INVALID      # dk aliases dq
    assert _bwd(lib, d=32) == _lib.FA_ERR_UNSUPPORTED
    assert _bwd(lib, do=None) == _lib.FA_ERR_INVALID


def test_fp8_rejects(lib):
    q = A
    assert lib.fa_quant_fp8(q, None, A + GAP, A + 2 * GAP, 1, 1, 64, 128, 32, 0, None) == _lib.FA_ERR_UNSUPPORTED
    assert lib.fa_quant_fp8(q, None, None, A + 2 * GAP, 1, 1, 64, 128, 64, 0, None) == _lib.FA_ERR_INVALID
    assert lib.fa_quant_fp8(q, None, A + 256, A + 2 * GAP, 1, 1, 64, 128, 64, 0, None) == _lib.FA_ERR_INVALID
    assert lib.fa_quant_fp8(q, None, A + GAP, A + 2 * GAP, 1, 1, 64, 128, 64, 2, None) == _lib.FA_ERR_INVALID
    s = A + 3 * GAP
    assert lib.fa_fwd_fp8(A, A + GAP, A + 2 * GAP, s, s + GAP, s + 2 * GAP, 64, s + 3 * GAP, s + 4 * GAP,
                          1, 1, 64, 64, 0.125, 0, None) == _lib.FA_ERR_UNSUPPORTED
    assert lib.fa_fwd_fp8(A, A + GAP, A + 2 * GAP, s, s + GAP, s + 2 * GAP, 64, A + 256, s + 4 * GAP,
                          1, 1, 64, 128, 0.125, 0, None) == _lib.FA_ERR_INVALID
    # scale blocks other than 64 rows (or one per tensor) are not supported
    for br in (32, 128, -1):
        assert lib.fa_fwd_fp8(A, A + GAP, A + 2 * GAP, s, s + GAP, s + 2 * GAP, br, s + 3 * GAP, s + 4 * GAP,
                              1, 1, 64, 128, 0.125, 0, None) == _lib.FA_ERR_UNSUPPORTED
        assert "block_rows" in lib.fa_last_error().decode()
        assert lib.fa_dequant_fp8(A, s, br, A + GAP, 1, 1, 64, 128, None) == _lib.FA_ERR_UNSUPPORTED
    assert lib.fa_dequant_fp8(A, s, 64, A + 8, 1, 1, 64, 128, None) == _lib.FA_ERR_UNSUPPORTED   # misaligned
    assert lib.fa_dequant_fp8(A, s, 64, A + 256, 1, 1, 64, 128, None) == _lib.FA_ERR_INVALID     # overlap
    assert lib.fa_dequant_fp8(A, None, 64, A + GAP, 1, 1, 64, 128, None) == _lib.FA_ERR_INVALID


def _bwd_fp8(lib, ws=A + 20 * GAP, ws_bytes=None, B=1, H=1, N=64, d=128, block_rows=64, **over):
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_fp8_workspace_bytes(B, H, N, d)
    p = {n: A + i * GAP for i, n in enumerate(("q8", "k8", "v8", "sq", "sk", "sv", "o", "lse", "do",
                                                 "dq", "dk", "dv"))}
    p.update(over)
    return lib.fa_bwd_fp8(p["q8"], p["k8"], p["v8"], p["sq"], p["sk"], p["sv"], block_rows, p["o"], p["lse"],
                          p["do"], p["dq"], p["dk"], p["dv"], ws, ws_bytes, B, H, N, d, 0.125, 1, None)


def test_fp8_backward_rejects_and_workspace(lib):
    B, H, N, d = 2, 3, 100, 128
    base = lib.fa_bwd_workspace_bytes(B, H, N, d)
    tb = -(-(B * H * N * d * 2) // 256) * 256
    assert lib.fa_bwd_fp8_workspace_bytes(B, H, N, d) == base + 3 * tb
    assert lib.fa_bwd_fp8_workspace_bytes(0, H, N, d) == 0
    assert _bwd_fp8(lib, ws=None) == _lib.FA_ERR_INVALID
    assert _bwd_fp8(lib, ws_bytes=100) == _lib.FA_ERR_INVALID
    assert _bwd_fp8(lib, ws=A + 20 * GAP + 16) == _lib.FA_ERR_UNSUPPORTED
    assert _bwd_fp8(lib, block_rows=32) == _lib.FA_ERR_UNSUPPORTED
    assert _bwd_fp8(lib, d=32) == _lib.FA_ERR_UNSUPPORTED
    assert _bwd_fp8(lib, dq=A + 256) == _lib.FA_ERR_INVALID          # dq overlaps q8
    assert _bwd_fp8(lib, dk=A + 9 * GAP) == _lib.FA_ERR_INVALID      # dk aliases dq
    assert _bwd_fp8(lib, sv=None) == _lib.FA_ERR_INVALID
    assert lib.fa_last_error()


def test_det_workspace_is_linear_in_n(lib):
    """The fixed-order backward keeps the method's O(N) extra memory ("6.1
    FlashAttention V1详解", 6.3): the plain backward's workspace (the float32
    dQ accumulator and D), plus 4 int32 counters per 32-row query tile and an
    error flag; the same for both masks."""
    def al(x):
        return (x + 255) // 256 * 256
    for (B, H, N, d, causal) in [(1, 1, 1, 64, 0), (1, 1, 1, 64, 1), (2, 3, 1000, 128, 1), (2, 3, 1000, 64, 0),
                                 (1, 2, 257, 128, 1), (1, 32, 16384, 128, 1), (1, 32, 16384, 128, 0)]:
        got = lib.fa_bwd_det_workspace_bytes(B, H, N, d, causal)
        counters = al(4 * (B * H * (-(-N // 32)) * 4 + 1))
        assert got == al(4 * B * H * N * d) + al(4 * B * H * N) + counters, (B, H, N, d, causal)
        assert got == lib.fa_bwd_workspace_bytes(B, H, N, d) + counters
    # linear in N: doubling N (a multiple of 32) doubles every part but the flag
    for N in (1024, 4096, 16384):
        one, two = (lib.fa_bwd_det_workspace_bytes(1, 32, n, 128, 1) for n in (N, 2 * N))
        assert abs(two - 2 * one) <= 512
    assert lib.fa_bwd_det_workspace_bytes(1, 32, 16384, 128, 0) == lib.fa_bwd_det_workspace_bytes(1, 32, 16384, 128, 1)
    # about 4 (d + 1) + 0.5 bytes per row: 270.6 MB at B=1, H=32, N=16384, d=128
    assert lib.fa_bwd_det_workspace_bytes(1, 32, 16384, 128, 1) < 271e6
    assert lib.fa_bwd_det_workspace_bytes(0, 1, 1, 64, 0) == 0
    assert lib.fa_bwd_det_workspace_bytes(1, 1, 1, 100, 1) == 0


def _bwd_det(lib, ws=A + 10 * GAP, ws_bytes=None, B=1, H=1, N=16, d=64, scale=0.125, causal=1, **over):
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_det_workspace_bytes(B, H, N, d, causal)
    p = dict(q=A, k=A + GAP, v=A + 2 * GAP, o=A + 3 * GAP, lse=A + 4 * GAP, do=A + 5 * GAP,
             dq=A + 6 * GAP, dk=A + 7 * GAP, dv=A + 8 * GAP)
    p.update(over)
    return lib.fa_bwd_det(p["q"], p["k"], p["v"], p["o"], p["lse"], p["do"], p["dq"], p["dk"], p["dv"],
                          ws, ws_bytes, B, H, N, d, scale, causal, None)


def test_det_backward_rejects(lib):
    assert _bwd_det(lib, ws=None) == _lib.FA_ERR_INVALID
    assert _bwd_det(lib, ws=A + 10 * GAP + 16) == _lib.FA_ERR_UNSUPPORTED
    # the plain backward's (smaller) workspace is not enough
    N = 1000
    small = lib.fa_bwd_workspace_bytes(1, 1, N, 64)
    assert small < lib.fa_bwd_det_workspace_bytes(1, 1, N, 64, 1)
    assert _bwd_det(lib, N=N, ws_bytes=small) == _lib.FA_ERR_INVALID
    assert "fa_bwd_det_workspace_bytes" in lib.fa_last_error().decode()
    # one byte short of the size
    assert _bwd_det(lib, N=N, ws_bytes=lib.fa_bwd_det_workspace_bytes(1, 1, N, 64, 1) - 1) == _lib.FA_ERR_INVALID
    assert _bwd_det(lib, dq=A + 64) == _lib.FA_ERR_INVALID
    assert _bwd_det(lib, d=32) == _lib.FA_ERR_UNSUPPORTED
    assert _bwd_det(lib, scale=float("nan")) == _lib.FA_ERR_UNSUPPORTED


def test_gqa_rejects(lib):
    def fwd(H=4, H_kv=2, N=16, d=64, **over):
        p = dict(q=A, k=A + GAP, v=A + 2 * GAP, o=A + 3 * GAP, lse=A + 4 * GAP)
        p.update(over)
        return lib.fa_fwd_gqa(p["q"], p["k"], p["v"], p["o"], p["lse"], 1, H, H_kv, N, d, 0.125, 1, None)

    def bwd(H=4, H_kv=2, N=16, d=64, ws_bytes=None):
        if ws_bytes is None:
            ws_bytes = max(lib.fa_bwd_gqa_workspace_bytes(1, H, max(H_kv, 1), N, d), 1 << 20)
        return lib.fa_bwd_gqa(A, A + GAP, A + 2 * GAP, A + 3 * GAP, A + 4 * GAP, A + 5 * GAP, A + 6 * GAP,
                              A + 7 * GAP, A + 8 * GAP, A + 10 * GAP, ws_bytes, 1, H, H_kv, N, d, 0.125, 1, None)

    for H_kv in (0, -1, 3, 5, 8):
        assert fwd(H_kv=H_kv) == _lib.FA_ERR_INVALID, H_kv
        assert "H_kv" in lib.fa_last_error().decode()
        assert bwd(H_kv=H_kv) == _lib.FA_ERR_INVALID, H_kv
    assert fwd(d=96) == _lib.FA_ERR_UNSUPPORTED
    assert fwd(o=A + 256) == _lib.FA_ERR_INVALID          # o overlaps q
    assert fwd(o=A + GAP + 64) == _lib.FA_ERR_INVALID     # o inside k
    assert bwd(ws_bytes=100) == _lib.FA_ERR_INVALID


def test_gqa_workspace(lib):
    def al(x):
        return (x + 255) // 256 * 256

    for (B, H, H_kv, N, d) in [(1, 32, 8, 16384, 128), (1, 32, 1, 16384, 128), (8, 32, 8, 16384, 128),
                               (2, 6, 3, 100, 64), (1, 4, 4, 300, 128)]:
        got = lib.fa_bwd_gqa_workspace_bytes(B, H, H_kv, N, d)
        base = lib.fa_bwd_workspace_bytes(B, H, N, d)
        # float32 dK and dV per query head when K/V heads are shared
        assert got == base + (al(2 * B * H * N * d * 4) if H_kv < H else 0), (B, H, H_kv, N, d)
    assert lib.fa_bwd_gqa_workspace_bytes(1, 6, 4, 100, 64) == 0
    assert lib.fa_bwd_gqa_workspace_bytes(1, 6, 0, 100, 64) == 0


def test_varlen_rejects_and_workspace(lib):
    def al(x):
        return (x + 255) // 256 * 256
    assert lib.fa_bwd_varlen_workspace_bytes(1000, 4, 4, 128) == lib.fa_bwd_workspace_bytes(1, 4, 1000, 128)
    assert lib.fa_bwd_varlen_workspace_bytes(1000, 4, 2, 64) == \
        lib.fa_bwd_workspace_bytes(1, 4, 1000, 64) + al(2 * 4 * 1000 * 64 * 4)
    assert lib.fa_bwd_varlen_workspace_bytes(1000, 4, 3, 64) == 0
    cu = A + 9 * GAP

    def fwd(n_seq=3, max_seqlen=100, total=300, H=4, H_kv=2, d=64, **over):
        p = dict(q=A, k=A + GAP, v=A + 2 * GAP, o=A + 3 * GAP, lse=A + 4 * GAP, cu=cu)
        p.update(over)
        return lib.fa_fwd_varlen(p["q"], p["k"], p["v"], p["o"], p["lse"], p["cu"], n_seq, max_seqlen, total,
                                 H, H_kv, d, 0.125, 1, None)

    def bwd(n_seq=3, max_seqlen=100, total=300, H=4, H_kv=2, d=64, ws_bytes=None, **over):
        p = dict(cu=cu, dq=A + 6 * GAP)
        p.update(over)
        if ws_bytes is None:
            ws_bytes = max(lib.fa_bwd_varlen_workspace_bytes(total, H, max(H_kv, 1), d), 1 << 20)
        return lib.fa_bwd_varlen(A, A + GAP, A + 2 * GAP, A + 3 * GAP, A + 4 * GAP, A + 5 * GAP, p["dq"],
                                 A + 7 * GAP, A + 8 * GAP, A + 10 * GAP, ws_bytes, p["cu"], n_seq, max_seqlen,
                                 total, H, H_kv, d, 0.125, 1, None)

    for call in (fwd, bwd):
        assert call(n_seq=0) == _lib.FA_ERR_INVALID
        assert call(max_seqlen=0) == _lib.FA_ERR_INVALID
        assert call(max_seqlen=301) == _lib.FA_ERR_INVALID        # longer than the packed batch
        assert call(H_kv=3) == _lib.FA_ERR_INVALID
        assert call(H_kv=0) == _lib.FA_ERR_INVALID
        assert call(d=96) == _lib.FA_ERR_UNSUPPORTED
        assert call(cu=None) == _lib.FA_ERR_INVALID
        assert call(cu=cu + 2) == _lib.FA_ERR_UNSUPPORTED         # misaligned
    assert fwd(o=cu) == _lib.FA_ERR_INVALID                        # output over cu_seqlens
    assert bwd(dq=cu) == _lib.FA_ERR_INVALID
    assert bwd(ws_bytes=1000) == _lib.FA_ERR_INVALID


def test_noalloc_backward_rejects(lib):
    """fa_bwd_noalloc checks its arguments before it looks up its scratch
    array, and refuses a head whose workspace exceeds that array."""
    assert lib.fa_bwd_noalloc_scratch_bytes() == 128 << 20

    def call(N=16, d=64, B=1, H=1, scale=0.125, **over):
        p = dict(q=A, k=A + GAP, v=A + 2 * GAP, o=A + 3 * GAP, lse=A + 4 * GAP, do=A + 5 * GAP,
                 dq=A + 6 * GAP, dk=A + 7 * GAP, dv=A + 8 * GAP)
        p.update(over)
        return lib.fa_bwd_noalloc(p["q"], p["k"], p["v"], p["o"], p["lse"], p["do"], p["dq"], p["dk"], p["dv"],
                                  B, H, N, d, scale, 1, None)
    assert call(B=0) == _lib.FA_ERR_INVALID
    assert call(d=32) == _lib.FA_ERR_UNSUPPORTED
    assert call(q=None) == _lib.FA_ERR_INVALID
    assert call(dq=A + 64) == _lib.FA_ERR_INVALID
    # one head of N = 300000, d = 128 needs about 155 MB of workspace
    assert call(N=300000, d=128) == _lib.FA_ERR_UNSUPPORTED
    assert "scratch" in lib.fa_last_error().decode()

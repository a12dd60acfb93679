"""ctypes loader for libfa_mi355x.so (the C ABI declared in include/fa.h).

Loading the library needs no GPU; calling a compute entry point does. There
is no fallback: if the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa_mi355x.so")

FA_OK = 0
FA_ERR_INVALID = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_HIP = -3

_c_int, _c_float, _c_size, _p = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/fa.h
SIGNATURES = {
    "fa_fwd": (_c_int, [_p, _p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _p]),
    "fa_fwd_f32": (_c_int, [_p, _p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _p]),
    "fa_bwd_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int]),
    "fa_bwd": (_c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _c_size,
                        _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _p]),
    "fa_bwd_stages": (_c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _c_size,
                               _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _c_int, _p]),
    "fa_fwd_gqa": (_c_int, [_p, _p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _p]),
    "fa_bwd_gqa": (_c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _c_size,
                            _c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _p]),
    "fa_bwd_gqa_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "fa_fwd_varlen": (_c_int, [_p, _p, _p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                               _c_float, _c_int, _p]),
    "fa_bwd_varlen": (_c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _c_size, _p,
                               _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _p]),
    "fa_bwd_varlen_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int]),
    "fa_bwd_det": (_c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _c_size,
                            _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _p]),
    "fa_bwd_det_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "fa_bwd_noalloc": (_c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p,
                                _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _p]),
    "fa_bwd_noalloc_scratch_bytes": (_c_size, []),
    "fa_bwd_f32": (_c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _c_size,
                            _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _p]),
    "fa_quant_fp8": (_c_int, [_p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _p]),
    "fa_fwd_fp8": (_c_int, [_p, _p, _p, _p, _p, _p, _c_int, _p, _p,
                            _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _p]),
    "fa_dequant_fp8": (_c_int, [_p, _p, _c_int, _p, _c_int, _c_int, _c_int, _c_int, _p]),
    "fa_bwd_fp8_workspace_bytes": (ctypes.c_size_t, [_c_int, _c_int, _c_int, _c_int]),
    "fa_bwd_fp8": (_c_int, [_p, _p, _p, _p, _p, _p, _c_int, _p, _p, _p, _p, _p, _p, _p, ctypes.c_size_t,
                            _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _p]),
    "fa_status_string": (ctypes.c_char_p, [_c_int]),
    "fa_last_error": (ctypes.c_char_p, []),
}

_lock = threading.Lock()
_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load(path: str = LIB_PATH):
    """Load the library once and attach the C signatures."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise FAError(FA_ERR_HIP, f"HIP library {path} is not built; run "
                          "`python -m exact_tiled_attention_12_amd.build` (or __graft_entry__.build())")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def check(status: int, what: str) -> None:
    if status != FA_OK:
        lib = load()
        detail = lib.fa_last_error().decode(errors="replace")
        kind = lib.fa_status_string(status).decode()
        raise FAError(status, f"{what}: {kind}: {detail}")

"""MI355X (gfx950) fused exact attention: a C-ABI HIP library plus this binding.

    from exact_tiled_attention_12_amd import fwd, bwd, quant_fp8, fwd_fp8

The binding only marshals torch tensors and the current HIP stream into the C
calls of include/fa.h; all computation runs in the library's kernels. The
library is built in-tree by ``python -m exact_tiled_attention_12_amd.build``.
"""

from ._lib import FAError, LIB_PATH, load  # noqa: F401


def __getattr__(name):
    if name in ("fwd", "bwd", "bwd_stages", "bwd_workspace_bytes", "bwd_det_workspace_bytes",
                "bwd_gqa_workspace_bytes", "fwd_varlen", "bwd_varlen", "quant_fp8", "fwd_fp8", "dequant_fp8",
                "bwd_fp8", "bwd_fp8_workspace_bytes"):
        from . import api
        return getattr(api, name)
    raise AttributeError(name)

"""Float64 CPU oracle for fused exact attention.

TEST INFRASTRUCTURE. Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package. The HIP library and its Python binding never import it, and it
imports nothing from them: the two share no code. The only module both sides
use is ``seeded_inputs`` (random draws, no attention arithmetic).

Modules:
  attention  plain definition: S, three-pass safe softmax, P V, LSE; backward
  online     tiled online-softmax recurrence (self-tests of the tiling only)
  fp8        e4m3 codec, block quantisation, tiled fp8 attention emulation

Every function is pinned by tests/test_oracle_*.py against values the pages
print, closed forms, brute force on tiny inputs, finite differences and CPU
library routines. No function here is "parity unpinned".
"""

from . import attention, online, fp8  # noqa: F401

"""The oracle: plain, slow, float64 CPU attention used to check the HIP path.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or run anything here. The HIP
library and its Python binding never touch this package, and this package imports
nothing from them. Its own correctness is pinned by the ``not gpu`` tests
(closed forms, invariants, brute force, finite differences, the pages' recurrences
and torch's CPU float64 attention).

Modules:
  attention  exact forward/backward from the definition (numpy float64)
  online     the pages' block recurrences (v1 normalised, v2 deferred)
  scalar     brute force with Python floats, math.fsum and math.exp
  fp8        E4M3 decoding, the FP8 forward's reference and its weight-rounding bound
"""
from . import attention, fp8, online, scalar  # noqa: F401

"""CPU float64 oracle for the fused attention forward.

TEST INFRASTRUCTURE ONLY. This package is the independent reference the HIP
path is checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product library never
does, and this package shares no code, header, table or helper with it.

Modules
-------
attention : plain materialised attention (scores, mods, mask, softmax, P.V)
            and a tiled online-softmax variant used only as an invariant.
fp8       : OCP e4m3 codec, Sylvester-Hadamard rotation with random signs,
            per-tile quantisation and an fp8 emulation of the attention.
"""
from . import attention, fp8  # noqa: F401

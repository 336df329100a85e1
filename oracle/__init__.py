"""Plain fp64 CPU oracle for attention forward/backward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP library.
"""
from .attention import (  # noqa: F401
    forward,
    forward_head,
    backward,
    backward_head,
    forward_rows_head,
    backward_q_rows_head,
    backward_kv_rows_head,
    reference,
    head_dropout,
)
from . import philox  # noqa: F401

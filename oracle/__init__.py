"""CPU oracle for MoE routing with load-balancing statistics.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the product path.
"""
from .oracle import (capacity, gate_logits, route, backward, bias_update,  # noqa: F401
                     load_library)

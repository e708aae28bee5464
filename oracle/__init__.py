"""CPU oracle for MoE routing with load-balancing statistics.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the product path.
"""
from .oracle import (capacity, gate_logits, gate_backward, route, backward,  # noqa: F401
                     bias_update, eplb, sinkhorn, load_library)

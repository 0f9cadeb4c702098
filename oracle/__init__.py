"""fp64 CPU oracle for chunkwise KDA prefill (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg
may import this package. The product path (the HIP library and its binding) never
does, and shares no code with it.
"""
from .kda_oracle import (  # noqa: F401
    L2_EPS, chunk_indices, kda_forward, kda_sequence, l2_normalize, sigmoid,
)

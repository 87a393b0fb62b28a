"""Seeded synthetic workloads for the CoW paged KV cache.

This package holds only input preparation: the shapes of each workload, the
operation trace (create / fork / append / free) that builds its tree of
sequences, and the seeded random draws that fill it. It contains none of the
method's arithmetic (no block tables, no refcounts, no attention). Both the
CPU oracle and the HIP path consume exactly these inputs.
"""

from .configs import (  # noqa: F401
    Op,
    Shape,
    Workload,
    WORKLOADS,
    get,
    scaled,
)
from .gen import Inputs, bf16_round, bf16_to_f32, generate, verify_parents  # noqa: F401

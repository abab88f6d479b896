"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This package holds the workload shapes and the seeded generators only; it
contains none of the method's arithmetic (no SVD, allocation, projection,
quantisation or attention).  Both the HIP path and the CPU oracle consume the
tensors it produces; neither imports the other.
"""
from .configs import CONFIGS, Config, pool_layout  # noqa: F401
from .planted import (  # noqa: F401
    derive_seed,
    planted_blocks,
    queries,
    selection,
    layer_inputs,
    tail_inputs,
)

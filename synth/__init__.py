"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This package holds no attention arithmetic: only workload sizes (``configs``)
and the random draws that fill Q, K, V and the per-head parameters
(``inputs``).  Both the fp64 oracle and the GPU path consume what it returns.
"""
from .configs import WORKLOADS, Workload, HEAD_SWA, HEAD_RETRIEVAL, HEAD_TRIANGLE, HEAD_DENSE  # noqa: F401
from .inputs import (  # noqa: F401
    bf16_round, make_layer_inputs, LayerInputs, gen_rows, gen_param,
)

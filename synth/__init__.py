"""Seeded synthetic inputs shaped like the workloads the WUSH pages evaluate on.

This module holds no arithmetic of the method: it only draws weights and
activations (numpy ``default_rng([config_id, stream])``) and rounds them to the
storage dtype.  Both the oracle-side tests and the GPU-side tests draw their
inputs from here.
"""

from .gen import CONFIGS, Workload, make_weights, make_activations, bf16_round, bf16_bits  # noqa: F401

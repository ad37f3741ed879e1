"""Seeded synthetic inputs for Parallax attention runs.

This package is shared by the GPU path's tests/bench and by the fp64 oracle's
tests. It draws random tensors and builds the probe input rho from a random
projection followed by an RMSNorm (the probe construction that the method
places before attention); it contains none of the attention arithmetic itself.
"""
from .inputs import (  # noqa: F401
    CONFIGS,
    DecodeConfig,
    PrefillConfig,
    decode_inputs,
    decode_grid_cells,
    prefill_head_inputs,
    prefill_inputs,
    prefill_upstream_grad,
    to_dtype,
)

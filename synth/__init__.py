"""Seeded synthetic inputs for the batched codec-LM decode step.

This package draws random tensors with the shapes and value distributions of
the five decode workloads and lays the KV history out in the paged pool format
that ``include/clm.h`` defines.  It holds none of the step's arithmetic
(no attention, projection, sampling or verification); both the CPU oracle's
tests and the GPU path's tests and benchmark take their inputs from here.
"""

from .configs import CONFIGS, DecodeConfig, get_config
from .gen import StepInputs, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs

__all__ = [
    "CONFIGS",
    "DecodeConfig",
    "get_config",
    "StepInputs",
    "make_inputs",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
]

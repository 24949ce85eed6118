"""Seeded synthetic inputs for the denoise step and the structured slot read.

This package only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both the CPU oracle (through the tests and the bench) and
the HIP path consume what it returns, so the two sides always see identical
inputs.
"""
from .configs import CONFIGS, Dims, config
from .generate import make_inputs, round_bf16, companion_row_scale, prompt_batch

__all__ = ["CONFIGS", "Dims", "config", "make_inputs", "round_bf16",
           "companion_row_scale", "prompt_batch"]

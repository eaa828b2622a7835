"""Seeded synthetic inputs for Sketch Attention compression.

This package is the only code shared by the fp64 oracle (``oracle/``) and the
GPU library's tests and bench.  It draws random numbers, rounds them to the
storage dtype and lays them out; it holds none of the method's arithmetic.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    Inputs,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_candidates,
    make_config,
    make_hard_assignment_inputs,
    make_inputs,
    make_sketch_grad,
    make_sketches,
)

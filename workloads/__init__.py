"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and
the benchmark.  This package holds input preparation only (random draws,
bf16 rounding of inputs, packing offsets); none of the method's arithmetic.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    as_f64,
    make_confidence,
    make_markov,
    make_repeated_markov,
    make_rnn,
    make_schedule,
    make_trees,
    make_tree_verify,
    make_verify_only,
    packed_offsets,
)

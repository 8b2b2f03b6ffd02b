"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.

This package holds input recipes only (shapes, value distributions, seeds and the
storage rounding of stored inputs). It computes nothing of the operator itself.
"""
from .inputs import (  # noqa: F401
    Hyena1DInputs,
    HyenaNDInputs,
    HyenaNDFilmInputs,
    CONFIGS,
    TEST_SHAPES,
    bf16_round,
    make_1d,
    make_nd,
    make_nd_film,
    make_config,
    sample_positions,
)

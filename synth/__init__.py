"""Seeded synthetic inputs (model shapes, random weights, random token streams).

This package is the only code shared by the CPU oracle and the HIP path. It holds
no model arithmetic: it describes shapes, draws seeded random numbers and lays
them out. Everything the RQ-Transformer computes lives elsewhere.
"""
from .moshi_inputs import (  # noqa: F401
    CONFIGS,
    MoshiConfig,
    bf16_round,
    config,
    param_count,
    raw_frames,
    weight_specs,
    generate_weights,
    generate_weight,
)
from . import mimi_inputs  # noqa: F401,E402

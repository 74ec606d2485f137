"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This package holds workload descriptions (shapes, sizes, distributions) and
random-number draws only. It performs none of the method's arithmetic: no
normalisation, projection, attention, schedule evaluation or token build.
"""
from .configs import CONFIGS, Config, PyramidRule, SemanticSpec, get_config
from .gen import (generate, make_weights, make_inputs, round_bf16, table_rows,
                  full_table, TABLE_BLOCK)

__all__ = [
    "CONFIGS", "Config", "PyramidRule", "SemanticSpec", "get_config",
    "generate", "make_weights", "make_inputs", "round_bf16", "table_rows",
    "full_table", "TABLE_BLOCK",
]

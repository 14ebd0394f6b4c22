"""Seeded synthetic workloads for MLA / GQLA decode.

This package holds the workload shapes and the seeded input generators shared by the
tests, the benchmark and the oracle's callers.  It holds none of the method's
arithmetic: only random draws, the paged-cache layout (page permutation, padding) and
the bf16 encoding of the drawn values.
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
from .gen import (make_inputs, make_append_inputs, make_projection_inputs,  # noqa: F401
                  bf16_round, Inputs)

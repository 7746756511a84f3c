"""Rounding of float64 values to the bf16 grid (nearest, ties to even).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Used where the method hands a computed vector on in bf16 (the serving setup of
"ReplaySSM: Cache SSM Inputs, Not State" keeps decode vectors in bf16): the fused
front-end's conv outputs and, when the ring is kept in bf16, the GDN corrections.
"""
from __future__ import annotations

import numpy as np


def round_bf16(x):
    """Nearest bf16 value of each float64 (8 significand bits, ties to even),
    returned as float64; finite inputs within the bf16 range."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                    # x = m * 2^e, 0.5 <= |m| < 1
    scaled = m * 256.0                    # 8 significand bits above the point
    return np.ldexp(np.round(scaled), e - 8)   # numpy rounds halves to even

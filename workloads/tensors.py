"""Seeded per-token tensors and the bfloat16 encoding of inputs.

Inputs are drawn in float32 and, for bfloat16 workloads, rounded to nearest
even into bfloat16 *once* here, so that both the oracle and the GPU path start
from the same exactly representable values.  bfloat16 arrays are carried as
their raw 16-bit patterns (``uint16``).
"""

from __future__ import annotations

import numpy as np


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to nearest-even bfloat16; returns uint16 bit
    patterns.  (Adding 0x7FFF plus the kept part's lowest bit to the 32-bit
    pattern carries into the kept 16 bits exactly when the dropped half is
    above one half, or equal to it with an odd kept part; for finite values
    the sum stays below 2^32.)"""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u >> 16
    r &= 1
    r += 0x7FFF
    r += u
    r >>= 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def draw_normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def sigmoid_f32(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)

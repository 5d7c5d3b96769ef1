"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds no attention arithmetic.  It only draws i.i.d. N(0, 1) values
with numpy's PCG64 generator and rounds fp32 to bf16 (round to nearest even), so
that the HIP path and the oracle receive bit-identical inputs: the GPU gets the
bf16 bits, the oracle gets the same values widened to fp64.
"""

from __future__ import annotations

import numpy as np

SEED_LAYOUT = 0x5EED
SEED_Q = 0x5EED + 1
SEED_K = 0x5EED + 2
SEED_V = 0x5EED + 3
SEED_DO = 0x5EED + 4


def normal_f32(seed: int, shape) -> np.ndarray:
    """i.i.d. standard normal float32 array from PCG64(seed)."""
    gen = np.random.Generator(np.random.PCG64(seed))
    return gen.standard_normal(size=shape, dtype=np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16, nearest-even; returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bf16 value, returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def make_tensor(seed: int, shape, dtype: str, std: float = 1.0):
    """Return (host_values_for_device, exact_values_f64).

    Values are N(0, std^2): the standard normal draw times ``std`` in float32,
    before any rounding.
    dtype "f32": device gets float32, oracle gets the same values in fp64.
    dtype "bf16": device gets uint16 bf16 bits, oracle gets their exact fp64 value.
    """
    x = normal_f32(seed, shape)
    if std != 1.0:
        x = x * np.float32(std)
    if dtype == "f32":
        return x, x.astype(np.float64)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x)
        return bits, bf16_bits_to_f32(bits).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")

"""bf16 <-> float64 for the oracle (test infrastructure only).

bf16 is the top half of an IEEE-754 binary32: 1 sign bit, 8 exponent bits, 7 mantissa bits.
Widening is exact: put the 16 bits in the high half of a binary32 and convert that to
float64.  Narrowing (used only to state what a correctly rounded bf16 result is) rounds the
float32 value to nearest, ties to even, on the 16 dropped bits.

Pins: widening is checked against hand-written bit patterns (1.0 = 0x3F80, -2.0 = 0xC000,
the smallest subnormal, +inf, NaN) and narrowing against ties and overflow cases in
tests/test_oracle_pins.py.
"""
import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """uint16 bf16 patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """float64 -> float32 (nearest even) -> bf16 (nearest even on the dropped 16 bits).

    NaN maps to the canonical quiet NaN 0x7FC0 with its sign kept.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lower = u & np.uint64(0xFFFF)
    upper = u >> np.uint64(16)
    half = np.uint64(0x8000)
    round_up = (lower > half) | ((lower == half) & ((upper & np.uint64(1)) == np.uint64(1)))
    out = (upper + round_up.astype(np.uint64)).astype(np.uint32)
    nan = np.isnan(f)
    sign = (u >> np.uint64(31)).astype(np.uint32) << np.uint32(15)
    out = np.where(nan, sign | np.uint32(0x7FC0), out)
    return out.astype(np.uint16)

"""Storage roundings of the path, float64 in and float64 out.

A merged proxy key is an fp32 sum, stored after two roundings: first to
bf16, then to E4M3; for scoring, the stored E4M3 value is converted exactly to
bf16 ("Step-5-Preview: Sparse Reads Are Not a Compressed KV Cache", sections
"Eight tokens become one search key, coordinate by coordinate" and
"Selection is a weighted ReLU score, not attention softmax").

* ``to_f32``     float64 -> nearest fp32 (ties to even), as a GPU fp32 result.
* ``round_bf16`` float64 -> fp32 -> bf16, both steps round-to-nearest-even.
* ``round_e4m3`` exact value -> OCP E4M3FN (bias 7, 3 mantissa bits,
  subnormal quantum 2**-9, largest finite 448, no infinities), nearest-even,
  saturating at +-448 (a reading: no page states the overflow rule, and the
  path's values stay far below 448).
* ``q8``         ``round_e4m3(round_bf16(x))``.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):          # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def to_f32(x: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest fp32 value (returned as float64)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> fp32 (RNE) -> bf16 (RNE) bit pattern."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32)).view(np.uint32)
    u = u.astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def round_bf16(x: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f64(f64_to_bf16_bits(x))


E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUBNORMAL_QUANTUM = 2.0 ** -9


def round_e4m3(x: np.ndarray) -> np.ndarray:
    """Nearest E4M3FN value (ties to even), saturating at +-448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # quantum of the binade: 2**(e-3) for normals, 2**-9 for subnormals
    _, e = np.frexp(np.where(a > 0, a, 1.0))      # a = m * 2**e, m in [0.5, 1)
    quantum = np.ldexp(1.0, (e - 1) - 3)
    quantum = np.where(a < E4M3_MIN_NORMAL, E4M3_SUBNORMAL_QUANTUM, quantum)
    r = np.rint(a / quantum) * quantum            # exact scaling, rint = ties-to-even
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, x)


def q8(x: np.ndarray) -> np.ndarray:
    """The store rounding: fp32 result -> BF16 -> E4M3, held as a bf16 value."""
    return round_e4m3(round_bf16(x))

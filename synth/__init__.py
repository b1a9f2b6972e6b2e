"""Seeded, counter-based synthetic inputs for the sparse GQA path.

This module is input infrastructure.  It holds none of the method's
arithmetic: it only turns (seed, tensor id, flat element index) into numbers.
Both the CPU oracle and the GPU path take their inputs from here, so a value
at a given index is the same on both sides:

* on the host, :func:`normal_f32`, :func:`normal_bf16_bits`,
  :func:`rms_rows_bf16_bits` and :func:`seq_lengths` compute any slice with
  NumPy;
* on the device, ``synth/gen.hip`` (loaded through :mod:`synth.device`)
  computes the same definition with integer operations and one correctly
  rounded fp32 multiply per value, and fills whole tensors in HBM.

Definition (every value is a pure function of its index):

1. ``h = splitmix64(seed ^ (tid << 48) ^ i)`` with the SplitMix64 output
   function of Steele, Lea and Flood, "Fast splittable pseudorandom number
   generators", OOPSLA 2014 (increment by the golden gamma, then the
   xor-shift-multiply finaliser).
2. ``S`` = sum of the four 16-bit lanes of ``h`` (an Irwin-Hall(4) draw on
   [0, 262140], mean 131070, variance 65536**2 / 3).
3. ``x = float32(S - 131070) * float32(c)`` rounded once to fp32, with
   ``c = sqrt(3) / 65536`` for unit variance (``c_w`` below for the indexer
   weights).  ``S - 131070`` is an exact integer below 2**24.
4. bf16 tensors round ``x`` to nearest-even on the bit pattern.
5. "RMS-normalised" bf16 rows (main Q and K): ``ss`` = sequential fp32 sum of
   the squares of the row's bf16 values, index 0 first (each square is exact
   in fp32), ``inv = 1 / sqrt(ss / width + 1e-6)`` with correctly rounded
   fp32 division and square root, value ``= bf16(x_bf16 * inv)``.

6. "Correlated" rows (an optional variant of the indexer queries and weights
   in which neighbouring query rows are alike): the value at (row r, column
   e) of a tensor of row width ``width`` is ``x = sum_j y_j`` over
   ``j = 0 .. W-1`` added in that order in fp32, with
   ``y_j = draw(tid, (r + W - 1 - j) * width + e)``, then ``x * c_W``
   rounded once, ``c_W = float32(1 / sqrt(W))`` (a moving sum of W
   independent draws: rows d apart share W - d of them, correlation
   (W - d) / W, and every value keeps the draws' variance).

Tensor ids: 1 Q, 2 K cache, 3 V cache, 4 indexer queries, 5 indexer weights,
6 proxy keys, 7 compression logits, 8 sequence lengths.
"""
from __future__ import annotations

import numpy as np

TID_Q = 1
TID_K = 2
TID_V = 3
TID_QIDX = 4
TID_W = 5
TID_PROXY = 6
TID_LOGITS = 7
TID_LEN = 8

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_MUL1 = np.uint64(0xBF58476D1CE4E5B9)
_MUL2 = np.uint64(0x94D049BB133111EB)
_MASK16 = np.uint64(0xFFFF)

#: unit-variance scale of the Irwin-Hall(4) draw, rounded once to fp32
C_UNIT = np.float32(np.sqrt(3.0) / 65536.0)
#: scale of the indexer weights: unit normal divided by sqrt(4 heads * 128 dims)
C_W = np.float32(np.sqrt(3.0) / 65536.0 / np.sqrt(512.0))
#: epsilon of the synthetic RMS normalisation of main Q / K rows
RMS_EPS = np.float32(1e-6)


def splitmix64(x: np.ndarray) -> np.ndarray:
    """SplitMix64 output function applied elementwise to uint64 ``x``."""
    x = np.asarray(x, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = x + _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _MUL1
        z = (z ^ (z >> np.uint64(27))) * _MUL2
        z = z ^ (z >> np.uint64(31))
    return z


def _hash(seed: int, tid: int, idx: np.ndarray) -> np.ndarray:
    base = np.uint64((int(seed) ^ (int(tid) << 48)) & 0xFFFFFFFFFFFFFFFF)
    return splitmix64(np.asarray(idx, dtype=np.uint64) ^ base)


def irwin_hall_centered(seed: int, tid: int, idx: np.ndarray) -> np.ndarray:
    """``S - 131070`` as int32 for each flat index."""
    h = _hash(seed, tid, idx)
    s = (h & _MASK16) + ((h >> np.uint64(16)) & _MASK16) \
        + ((h >> np.uint64(32)) & _MASK16) + (h >> np.uint64(48))
    return s.astype(np.int64).astype(np.int32) - np.int32(131070)


def normal_f32(seed: int, tid: int, idx: np.ndarray, scale: np.float32 = C_UNIT) -> np.ndarray:
    """fp32 values ``float32(S - 131070) * scale`` (one rounding)."""
    c = irwin_hall_centered(seed, tid, idx).astype(np.float32)
    return (c * np.float32(scale)).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16_bits(seed: int, tid: int, idx: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of unit-variance draws at flat indices ``idx``."""
    return f32_to_bf16_bits(normal_f32(seed, tid, idx))


def rms_rows_bf16_bits(seed: int, tid: int, rows: np.ndarray, width: int) -> np.ndarray:
    """RMS-normalised bf16 rows ``[len(rows), width]``; row ``r`` covers flat
    indices ``r*width .. r*width+width-1``."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    idx = rows[:, None] * np.int64(width) + np.arange(width, dtype=np.int64)[None, :]
    xb = normal_bf16_bits(seed, tid, idx.astype(np.uint64))
    x = bf16_bits_to_f32(xb)
    ss = np.zeros(rows.shape[0], dtype=np.float32)
    for j in range(width):           # fixed order: index 0 first
        ss = (ss + x[:, j] * x[:, j]).astype(np.float32)
    mean = (ss / np.float32(width)).astype(np.float32)
    inv = (np.float32(1.0) / np.sqrt((mean + RMS_EPS).astype(np.float32))).astype(np.float32)
    return f32_to_bf16_bits((x * inv[:, None]).astype(np.float32))


def seq_lengths(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """Per-sequence lengths, uniform on the integers [lo, hi]."""
    h = _hash(seed, TID_LEN, np.arange(n, dtype=np.uint64))
    span = np.uint64(hi - lo + 1)
    return (h % span).astype(np.int64) + np.int64(lo)


def corr_rows_f32(seed: int, tid: int, rows: np.ndarray, width: int, window: int,
                  scale: np.float32 = C_UNIT) -> np.ndarray:
    """Correlated rows ``[len(rows), width]`` (item 6 above): a moving sum of
    ``window`` draws along the row index, added in a fixed order."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    cols = np.arange(width, dtype=np.int64)[None, :]
    acc = np.zeros((rows.shape[0], width), dtype=np.float32)
    for j in range(window):
        idx = (rows[:, None] + np.int64(window - 1 - j)) * np.int64(width) + cols
        acc = (acc + normal_f32(seed, tid, idx.astype(np.uint64), scale)).astype(np.float32)
    c = np.float32(1.0 / np.sqrt(float(window)))
    return (acc * c).astype(np.float32)

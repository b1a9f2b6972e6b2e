"""Pins of the oracle's storage roundings against library casts and worked
examples (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import numerics as nu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_bf16(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _edge_f32():
    rng = np.random.default_rng(1)
    # random bit patterns over every binade (finite only)
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # exact bf16 midpoints (ties) and their neighbours
    base = rng.integers(0, 2**16, size=20_000, dtype=np.uint32) << np.uint32(16)
    mids = base | np.uint32(0x8000)
    near = np.concatenate([mids, mids + np.uint32(1), mids - np.uint32(1)])
    y = near.view(np.float32)
    y = y[np.isfinite(y)]
    special = np.array([0.0, -0.0, 1.0, -1.0, 1e-40, -1e-40, 3.0e38, 1.17549435e-38],
                       dtype=np.float32)
    return np.concatenate([x, y, special])


def test_bf16_matches_torch_cast():
    x = _edge_f32()
    ours = nu.f64_to_bf16_bits(x.astype(np.float64))
    ref = _torch_bf16(x)
    assert np.array_equal(ours, ref)


def test_bf16_two_step_from_f64():
    # float64 values are first rounded to fp32, as a GPU fp32 result would be
    rng = np.random.default_rng(2)
    x = rng.standard_normal(100_000) * np.exp2(rng.integers(-20, 20, 100_000))
    ours = nu.f64_to_bf16_bits(x)
    ref = _torch_bf16(x.astype(np.float32))
    assert np.array_equal(ours, ref)
    assert np.array_equal(nu.round_bf16(x), nu.bf16_bits_to_f64(ref))


def test_bf16_widen_exact():
    bits = np.arange(0, 2**16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = nu.bf16_bits_to_f64(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin], ref[fin])


def test_e4m3_matches_torch_on_all_bf16_in_range():
    bits = np.arange(0, 2**16, dtype=np.uint32).astype(np.uint16)
    x = nu.bf16_bits_to_f64(bits)
    x = x[np.isfinite(x) & (np.abs(x) <= 448.0)]
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = nu.round_e4m3(x)
    assert np.array_equal(ours, ref)
    # signs of zero follow the input
    assert np.array_equal(np.signbit(ours), np.signbit(ref))


def test_e4m3_matches_torch_on_random_f32():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(200_000) * np.exp2(rng.integers(-14, 9, 200_000))).astype(np.float32)
    x = x[np.abs(x) <= 448.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(nu.round_e4m3(x.astype(np.float64)), ref)


def test_e4m3_grid_and_saturation():
    # every E4M3FN finite value is a fixed point; 448 is the largest
    vals = torch.arange(0, 256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    v = vals.to(torch.float64).numpy()
    v = v[np.isfinite(v)]
    assert np.array_equal(nu.round_e4m3(v), v)
    assert v.max() == 448.0
    # saturation reading (no page states the overflow rule)
    assert nu.round_e4m3(np.array([500.0, -1e6]))[0] == 448.0
    assert nu.round_e4m3(np.array([500.0, -1e6]))[1] == -448.0
    # subnormal quantum 2**-9; 2**-10 is a tie with zero -> even -> 0
    assert nu.round_e4m3(np.array([2.0 ** -10]))[0] == 0.0
    assert nu.round_e4m3(np.array([1.5 * 2.0 ** -9]))[0] == 2.0 ** -8


def test_store_rounding_goes_through_bf16():
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        ex = json.load(f)["store_rounding_through_bf16"]
    x = np.array([ex["x"]])
    assert nu.round_bf16(x)[0] == ex["bf16"]
    assert nu.q8(x)[0] == ex["q8"]
    assert nu.round_e4m3(x)[0] == ex["direct_e4m3"]


def test_to_f32():
    x = np.array([1.0 + 2.0 ** -30, 0.1])
    assert np.array_equal(nu.to_f32(x), np.array([1.0, np.float32(0.1)], dtype=np.float64))

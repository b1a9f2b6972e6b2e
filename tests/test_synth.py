"""The seeded input generator: the published SplitMix64 sequence, the
Irwin-Hall draw's support and moments, bf16 rounding, RMS rows (CPU only)."""
import numpy as np
import torch

import synth


def test_splitmix64_published_sequence():
    # SplitMix64 seeded with 0 yields e220a8397b1dcdaf, 6e789e6aa1b965f4,
    # 06c45d188009454f (state advances by the golden gamma before mixing);
    # our counter form mixes (i + gamma), so state k*gamma is index (k-1)*gamma.
    g = np.uint64(0x9E3779B97F4A7C15)
    with np.errstate(over="ignore"):
        idx = np.array([0, g, g * np.uint64(2)], dtype=np.uint64)
    out = synth.splitmix64(idx)
    assert [int(v) for v in out] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_irwin_hall_support_and_moments():
    c = synth.irwin_hall_centered(0, synth.TID_V, np.arange(1 << 20, dtype=np.uint64))
    assert c.min() >= -131070 and c.max() <= 131070
    x = c.astype(np.float64) * float(synth.C_UNIT)
    assert abs(x.mean()) < 5e-3
    assert abs(x.std() - 1.0) < 5e-3
    # excess kurtosis of Irwin-Hall(4) is -0.3
    k = ((x - x.mean()) ** 4).mean() / x.var() ** 2 - 3.0
    assert abs(k + 0.3) < 0.03


def test_streams_are_independent_of_tensor_id():
    i = np.arange(4096, dtype=np.uint64)
    a = synth.normal_f32(0, synth.TID_Q, i)
    b = synth.normal_f32(0, synth.TID_K, i)
    assert abs(np.corrcoef(a, b)[0, 1]) < 0.06


def test_bf16_bits_match_torch():
    x = synth.normal_f32(7, synth.TID_PROXY, np.arange(100_000, dtype=np.uint64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.normal_bf16_bits(7, synth.TID_PROXY, np.arange(100_000, dtype=np.uint64)), ref)


def test_rms_rows_unit_rms_and_slice_consistency():
    rows = np.arange(300)
    full = synth.rms_rows_bf16_bits(0, synth.TID_K, rows, 192)
    x = synth.bf16_bits_to_f32(full).astype(np.float64)
    rms = np.sqrt((x * x).mean(axis=1))
    assert np.all(np.abs(rms - 1.0) < 1e-2)
    # any subset of rows regenerates bit-identically
    sub = synth.rms_rows_bf16_bits(0, synth.TID_K, rows[[5, 17, 299]], 192)
    assert np.array_equal(sub, full[[5, 17, 299]])


def test_seq_lengths_range():
    L = synth.seq_lengths(0, 64, 131072, 262144)
    assert L.min() >= 131072 and L.max() <= 262144
    assert len(set(L.tolist())) == 64


def test_group_slices_equal_full_rows():
    from synth import workloads as W
    wl = W.make("prefill_8k")
    rows = np.array([0, 5, 77, 8191, 3000])
    k, v = W.host_k(wl, rows), W.host_v(wl, rows)
    for g in range(4):
        assert np.array_equal(k[:, g], W.host_k_group(wl, rows, g))
        assert np.array_equal(v[:, g], W.host_v_group(wl, rows, g))


def test_correlated_rows_are_moving_sums():
    """Item 6 of the generator: each value is the sum of `window` draws at the
    documented indices (checked in float64 against the fp32 result within
    its rounding), neighbouring rows share draws, and the variance is kept."""
    W_, width = 16, 24
    rows = np.array([0, 1, 5, 900], dtype=np.int64)
    got = synth.corr_rows_f32(7, synth.TID_QIDX, rows, width, W_)
    for a, r in enumerate(rows):
        idx = ((r + W_ - 1 - np.arange(W_))[:, None] * width + np.arange(width)[None, :]).astype(np.uint64)
        ref = synth.normal_f32(7, synth.TID_QIDX, idx).astype(np.float64).sum(axis=0) / np.sqrt(W_)
        assert np.allclose(got[a], ref, rtol=0, atol=1e-5)
    many = synth.corr_rows_f32(7, synth.TID_QIDX, np.arange(4000), 64, W_)
    assert abs(float(many.std()) - 1.0) < 0.03
    d1 = np.mean([np.corrcoef(many[i], many[i + 1])[0, 1] for i in range(0, 3900, 50)])
    d8 = np.mean([np.corrcoef(many[i], many[i + 8])[0, 1] for i in range(0, 3900, 50)])
    assert abs(d1 - (W_ - 1) / W_) < 0.05 and abs(d8 - (W_ - 8) / W_) < 0.08

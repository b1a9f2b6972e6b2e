"""Comparison rules between the HIP path and the CPU oracle.

The oracle computes from the same seeded inputs on its own (nothing it reads
comes from the GPU).  Three places admit more than one correct result, and
for them the rules below compare what is unique and check that the rest is
valid:

1. Storage roundings (the bf16 indexer query, the bf16 / E4M3 summaries).
   The GPU rounds an fp32 value, the oracle a float64 one; when the exact
   value sits within the fp32 computation error of a rounding boundary either
   neighbour is correct.  Rule: the GPU value must lie in
   [fmt(x - a), fmt(x + a)] with a = REL * max(|x|, 1) (fmt is monotone), so
   away from boundaries the match is exact.
2. Scores.  From the admissible intervals of q_hat and of the summaries,
   interval arithmetic bounds every score (plus the fp32 accumulation error of
   the 128-term dot product).  GPU scores must lie in the bound widened by the
   1e-3 relative score tolerance.
3. Selection.  The GPU's set must be a valid top-k for some admissible
   rounding: no chosen block may be clearly worse than an unchosen one (beyond
   the 1e-4 relative tie band around the k-th score), exact ties must go to
   the lower block id, counts must match, ids ascending and causal.  Where the
   GPU set equals the oracle's, attention is compared against the oracle's
   output; where it differs but is valid, against the oracle's attention over
   the GPU's (validated) set.

Attention outputs, per (query row, head) vector of 192 values: the relative
error ||diff|| / ||ref|| <= 1e-2 and every element within 2e-2 * max |ref| of
that vector, besides max |diff| <= 2e-2 over everything compared; the
log-sum-exp within 1e-3 absolute.  A single ratio over all rows stacked would
be dominated by the early rows (fewer than B tokens attended, outputs near 1)
and would let a large error on the long rows (outputs near 0.02) through.
"""
from __future__ import annotations

import numpy as np

from oracle import numerics as nu

REL_STORE = 2.0 ** -17
REL_QHAT = 2.0 ** -17
ACC_REL = 2.0 ** -18          # fp32 accumulation bound on a 128-term dot, per |q||S|
SCORE_REL = 1e-3
TIE_REL = 1e-4
O_MAX_ABS = 2e-2
O_REL_FRO = 1e-2
LSE_ABS = 1e-3


def bits_to_f64(bits) -> np.ndarray:
    return nu.bf16_bits_to_f64(np.asarray(bits).view(np.uint16))


def rounding_interval(exact: np.ndarray, q8: bool, rel: float):
    fmt = nu.q8 if q8 else nu.round_bf16
    a = rel * np.maximum(np.abs(exact), 1.0)
    return fmt(exact - a), fmt(exact + a)


def check_rounded(gpu_vals: np.ndarray, exact: np.ndarray, q8: bool, rel: float, what: str,
                  max_excused_frac: float = 2e-3) -> dict:
    """Every GPU value within its admissible interval; report how many
    differ from the oracle's own rounding."""
    lo, hi = rounding_interval(exact, q8, rel)
    ok = (gpu_vals >= lo) & (gpu_vals <= hi)
    ref = nu.q8(exact) if q8 else nu.round_bf16(exact)
    bad = np.argwhere(~ok)
    assert bad.size == 0, (
        f"{what}: {bad.shape[0]} of {ok.size} values outside the admissible rounding interval; "
        f"first at {bad[0].tolist()}: gpu={gpu_vals[tuple(bad[0])]!r} "
        f"exact={exact[tuple(bad[0])]!r} oracle={ref[tuple(bad[0])]!r}")
    excused = int(np.count_nonzero(gpu_vals != ref))
    assert excused <= max_excused_frac * gpu_vals.size + 2, f"{what}: {excused} boundary cases"
    diff = gpu_vals - ref
    return {"n": int(gpu_vals.size), "boundary_cases": excused,
            "max_abs": float(np.abs(diff).max()) if diff.size else 0.0}


class StoreBounds:
    """Midpoints and radii of the admissible store values [s_lo, s_hi]
    ([b, Di]), computed once per sequence so that bounding one (query, group)
    row costs only small matrix products."""

    def __init__(self, s_lo, s_hi):
        self.sc = (s_lo + s_hi) / 2
        self.sr = (s_hi - s_lo) / 2
        self.abs_sc = np.abs(self.sc)


def score_bounds(q_lo, q_hi, s_lo, s_hi, w, sb: StoreBounds = None, b: int = None):
    """Interval bounds of sum_i w_i relu(q_i . S_r) over admissible q in
    [q_lo, q_hi] ([Hi, Di]) and S in [s_lo, s_hi] ([b, Di]); returns
    (lo [b], hi [b]).  With `sb` (the store's precomputed midpoints and
    radii) the first `b` store rows are used and s_lo / s_hi are ignored."""
    qc, qr = (q_lo + q_hi) / 2, (q_hi - q_lo) / 2
    if sb is None:
        sb = StoreBounds(s_lo, s_hi)
        b = sb.sc.shape[0]
    sc, sr, abs_sc = sb.sc[:b], sb.sr[:b], sb.abs_sc[:b]
    dot = sc @ qc.T
    rad = abs_sc @ qr.T + sr @ np.abs(qc).T + sr @ qr.T
    rad = rad + ACC_REL * (abs_sc @ np.abs(qc).T) + 1e-30
    dl, dh = np.maximum(dot - rad, 0.0), np.maximum(dot + rad, 0.0)
    w = np.asarray(w, dtype=np.float64)[None, :]
    lo = np.where(w >= 0, w * dl, w * dh).sum(axis=1)
    hi = np.where(w >= 0, w * dh, w * dl).sum(axis=1)
    # a dot whose interval is exactly 0 on the clipped side is a certain zero
    return lo, hi


def check_selection(sel: np.ndarray, b: int, k: int, s_ref: np.ndarray, s_lo: np.ndarray,
                    s_hi: np.ndarray, where: str) -> None:
    n = min(k, b)
    sel = np.asarray(sel, dtype=np.int64)
    assert np.all(sel[n:] == -1), f"{where}: padding must be -1"
    chosen_ids = sel[:n]
    assert np.all(chosen_ids >= 0) and np.all(chosen_ids < b), f"{where}: id out of [0, {b})"
    assert np.all(np.diff(chosen_ids) > 0), f"{where}: ids not strictly ascending"
    if n == b:
        return
    chosen = np.zeros(b, dtype=bool)
    chosen[chosen_ids] = True
    sK = np.sort(s_ref)[::-1][k - 1]
    sigma = float(np.sqrt(np.mean(s_ref * s_ref)))
    tau = TIE_REL * max(abs(sK), sigma)
    worst_in = s_hi[chosen].min()
    best_out = s_lo[~chosen].max()
    assert worst_in >= best_out - tau, (
        f"{where}: chose block {int(np.flatnonzero(chosen)[np.argmin(s_hi[chosen])])} "
        f"(upper {worst_in!r}) over block {int(np.flatnonzero(~chosen)[np.argmax(s_lo[~chosen])])} "
        f"(lower {best_out!r}), band {tau!r}")
    # exact ties (degenerate intervals of equal value) go to the lower id
    deg = s_lo == s_hi
    vin = s_lo[deg & chosen]
    vout = s_lo[deg & ~chosen]
    for v in np.intersect1d(vin, vout):
        ids_in = np.flatnonzero(deg & chosen & (s_lo == v))
        ids_out = np.flatnonzero(deg & ~chosen & (s_lo == v))
        assert ids_in.max() < ids_out.min(), f"{where}: tie at {v} not resolved to lower ids"


def check_scores(gpu_scores: np.ndarray, sel: np.ndarray, s_ref, s_lo, s_hi, where: str) -> float:
    n = int(np.count_nonzero(sel >= 0))
    if n == 0:
        return 0.0
    ids = sel[:n]
    sigma = float(np.sqrt(np.mean(s_ref * s_ref))) if s_ref.size else 0.0
    tol = SCORE_REL * np.maximum(np.abs(s_ref[ids]), sigma)
    g = gpu_scores[:n].astype(np.float64)
    ok = (g >= s_lo[ids] - tol) & (g <= s_hi[ids] + tol)
    assert ok.all(), (f"{where}: score of block {int(ids[~ok][0])} gpu={g[~ok][0]!r} "
                      f"bounds=({s_lo[ids][~ok][0]!r}, {s_hi[ids][~ok][0]!r})")
    return float(np.max(np.abs(g - s_ref[ids]) / np.maximum(np.abs(s_ref[ids]), sigma + 1e-30)))


def check_attention(o_gpu: np.ndarray, o_ref: np.ndarray, lse_gpu=None, lse_ref=None,
                    what: str = "attention") -> dict:
    """o_* [..., D]: every vector along the last axis is one (row, head)
    output; lse_* the matching [...] log-sum-exps."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    assert o_gpu.shape == o_ref.shape, f"{what}: shapes {o_gpu.shape} vs {o_ref.shape}"
    d = (o_gpu - o_ref).reshape(-1, o_ref.shape[-1])
    r = o_ref.reshape(-1, o_ref.shape[-1])
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite outputs"
    max_abs = float(np.abs(d).max())
    assert max_abs <= O_MAX_ABS, f"{what}: max |diff| {max_abs} > {O_MAX_ABS}"
    vec_rel = np.linalg.norm(d, axis=1) / np.maximum(np.linalg.norm(r, axis=1), 1e-30)
    worst = int(np.argmax(vec_rel))
    assert vec_rel[worst] <= O_REL_FRO, (
        f"{what}: vector {worst} of {r.shape[0]}: ||diff|| / ||ref|| {vec_rel[worst]} > {O_REL_FRO}")
    scale = np.abs(r).max(axis=1)
    elem = np.abs(d).max(axis=1) / np.maximum(scale, 1e-30)
    worst_e = int(np.argmax(elem))
    assert elem[worst_e] <= O_MAX_ABS, (
        f"{what}: vector {worst_e}: max |diff| {np.abs(d[worst_e]).max()} above "
        f"{O_MAX_ABS} x max |ref| {scale[worst_e]}")
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(r), 1e-30))
    out = {"max_abs": max_abs, "rel_fro": rel, "vectors": int(r.shape[0]),
           "max_vec_rel": float(vec_rel[worst]), "max_elem_rel": float(elem[worst_e])}
    if lse_gpu is not None:
        lg = np.asarray(lse_gpu, dtype=np.float64)
        assert np.all(np.isfinite(lg)), f"{what}: non-finite log-sum-exp"
        dl = float(np.abs(lg - np.asarray(lse_ref, dtype=np.float64)).max())
        assert dl <= LSE_ABS, f"{what}: lse diff {dl} > {LSE_ABS}"
        out["lse_max_abs"] = dl
    return out

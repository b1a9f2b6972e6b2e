"""The comparison rules of tests/parity.py on constructed cases (CPU only):
they accept what a correct bf16 path produces and reject errors the old
stacked-tensor rule let through."""
import numpy as np
import pytest

from oracle import numerics as nu
from tests import parity as P


def _outputs(seed=0):
    """Reference outputs of 8 rows x 16 heads x 192 dims: two early rows with
    values near 1 (a handful of attended tokens) and six long rows near 0.02
    (a softmax over thousands of tokens)."""
    rng = np.random.default_rng(seed)
    o = rng.standard_normal((8, 16, 192))
    o[:2] *= 0.8
    o[2:] *= 0.02
    lse = rng.standard_normal((8, 16)) + 8.0
    return o, lse


def test_bf16_rounded_outputs_pass():
    o, lse = _outputs()
    got = nu.round_bf16(o)
    st = P.check_attention(got, o, lse + 1e-5, lse)
    assert st["max_vec_rel"] < 4e-3 and st["vectors"] == 128


def test_error_confined_to_long_rows_fails():
    # 15 % relative error on the long rows only: the early rows dominate a
    # stacked Frobenius ratio (about 2.4e-3 here), and the largest absolute
    # difference stays under 2e-2, so only the per-vector rule catches it
    o, lse = _outputs()
    bad = o.copy()
    bad[2:] *= 1.15
    d = bad - o
    assert np.abs(d).max() < P.O_MAX_ABS
    assert np.linalg.norm(d) / np.linalg.norm(o) < P.O_REL_FRO
    with pytest.raises(AssertionError, match="diff"):
        P.check_attention(bad, o)


def test_zeroed_long_rows_fail():
    o, _ = _outputs()
    bad = o.copy()
    bad[5] = 0.0
    with pytest.raises(AssertionError):
        P.check_attention(bad, o)


def test_one_wrong_element_in_a_long_row_fails():
    o, _ = _outputs()
    bad = nu.round_bf16(o)
    bad[4, 3, 17] += 0.05 * np.abs(o[4, 3]).max()
    with pytest.raises(AssertionError):
        P.check_attention(bad, o)


def test_lse_and_non_finite_outputs_fail():
    o, lse = _outputs()
    with pytest.raises(AssertionError, match="lse"):
        P.check_attention(o, o, lse + 2e-3, lse)
    bad = o.copy()
    bad[3, 0, 0] = np.nan
    with pytest.raises(AssertionError, match="non-finite"):
        P.check_attention(bad, o)

"""The parity checker itself (``tests.helpers.assert_parity``), on hand-made outputs: it must
pass an output that matches the reference, and fail on any non-finite value where the reference
is finite, on a wrong empty-token result, and on errors above the stated bar."""

import numpy as np
import pytest
import torch

from tests import helpers as th


def _ref(seed=0):
    rng = np.random.default_rng(seed)
    ref_o = rng.standard_normal((2, 3, 4, 512))
    ref_l = rng.standard_normal((2, 3, 4))
    return ref_o, ref_l


def _t(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float32))


def test_matching_output_passes_and_reports_small_errors():
    ref_o, ref_l = _ref()
    worst, worst_lse = th.assert_parity(_t(ref_o), _t(ref_l), ref_o, ref_l, what="exact")
    assert worst < 1e-6 and worst_lse < 1e-6


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_non_finite_output_fails(bad):
    ref_o, ref_l = _ref()
    out = ref_o.copy()
    out[1, 2, 3, 100] = bad
    with pytest.raises(AssertionError, match="non-finite"):
        th.assert_parity(_t(out), _t(ref_l), ref_o, ref_l, what="planted")


def test_all_nan_output_fails():
    ref_o, ref_l = _ref()
    with pytest.raises(AssertionError):
        th.assert_parity(_t(np.full_like(ref_o, np.nan)), _t(ref_l), ref_o, ref_l)


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_non_finite_lse_fails(bad):
    ref_o, ref_l = _ref()
    lse = ref_l.copy()
    lse[0, 1, 2] = bad
    with pytest.raises(AssertionError, match="lse"):
        th.assert_parity(_t(ref_o), _t(lse), ref_o, ref_l)


def test_empty_token_needs_zero_output_and_minus_inf():
    ref_o, ref_l = _ref()
    ref_o[1, 0] = 0.0
    ref_l[1, 0] = -np.inf
    th.assert_parity(_t(ref_o), _t(ref_l), ref_o, ref_l)            # exact empty result passes
    out = ref_o.copy()
    out[1, 0, 2, 5] = 1e-3
    with pytest.raises(AssertionError):
        th.assert_parity(_t(out), _t(ref_l), ref_o, ref_l)
    lse = ref_l.copy()
    lse[1, 0, 1] = 0.0                                                # finite lse for an empty token
    with pytest.raises(AssertionError, match="lse"):
        th.assert_parity(_t(ref_o), _t(lse), ref_o, ref_l)


def test_error_above_the_bar_fails_and_below_passes():
    ref_o, ref_l = _ref()
    out = ref_o.copy()
    m = np.max(np.abs(ref_o[0, 0, 0]))
    out[0, 0, 0, 7] += 3e-3 * m
    with pytest.raises(AssertionError, match="row relative error"):
        th.assert_parity(_t(out), _t(ref_l), ref_o, ref_l)
    out = ref_o.copy()
    out[0, 0, 0, 7] += 1e-3 * m
    th.assert_parity(_t(out), _t(ref_l), ref_o, ref_l)
    lse = ref_l.copy()
    lse[0, 0, 0] += 3e-3
    with pytest.raises(AssertionError, match="lse error"):
        th.assert_parity(_t(ref_o), _t(lse), ref_o, ref_l)


def test_only_listed_tokens_are_compared():
    ref_o, ref_l = _ref()
    out = ref_o.copy()
    out[1, 1] = np.nan                      # a token outside the list is not looked at
    th.assert_parity(_t(out), _t(ref_l), ref_o, ref_l, tokens=[(0, 0), (1, 2)])

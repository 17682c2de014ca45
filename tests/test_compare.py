"""Pins of the tolerance check that decides every GPU parity verdict
(oracle/compare.py::check), on hand-made arrays, no GPU.

The bar it implements: over the whole O tensor max|O_gpu - O_ref| <= 1e-2 and
||O_gpu - O_ref||_2 / ||O_ref||_2 <= 5e-3; |LSE_gpu - LSE_ref| <= 1e-3 where
the oracle's LSE is finite; where the oracle's selection is empty (LSE =
-inf) the GPU must give LSE = -inf and O == 0 exactly; no NaN anywhere.
Each rule is exercised on both sides of its threshold, so a slip in a mask,
a comparison or the rel-L2 normaliser fails here rather than passing a
wrong kernel.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle.compare import LSE_ABS, MAX_ABS, REL_L2, check

T, H, DV = 3, 4, 512


def ref():
    """A reference with every entry finite except token 2 / head 3 (empty)."""
    rng = np.random.default_rng(7)
    o = rng.normal(0.0, 1.0, (T, H, DV))
    lse = rng.uniform(5.0, 9.0, (T, H))
    o[2, 3] = 0.0
    lse[2, 3] = -np.inf
    return o, lse


def test_identical_passes():
    o, l = ref()
    ok, m = check(o.copy(), l.copy(), o, l)
    assert ok, m["reasons"]
    assert m["max_abs"] == 0.0 and m["rel_l2"] == 0.0 and m["lse_max_abs"] == 0.0
    assert m["empty"] == 1 and m["n"] == T * H * DV


@pytest.mark.parametrize("where", ["o", "lse"])
def test_nan_fails(where):
    o, l = ref()
    og, lg = o.copy(), l.copy()
    if where == "o":
        og[1, 2, 100] = np.nan
    else:
        lg[0, 1] = np.nan
    ok, m = check(og, lg, o, l)
    assert not ok and any("NaN" in r for r in m["reasons"])


def test_nan_in_an_empty_row_fails():
    o, l = ref()
    og, lg = o.copy(), l.copy()
    og[2, 3, 0] = np.nan
    assert not check(og, lg, o, l)[0]


def test_inf_in_o_fails():
    o, l = ref()
    og = o.copy()
    og[0, 0, 0] = np.inf
    assert not check(og, l.copy(), o, l)[0]


def test_lse_minus_inf_on_gpu_only_fails():
    o, l = ref()
    lg = l.copy()
    lg[1, 1] = -np.inf
    ok, m = check(o.copy(), lg, o, l)
    assert not ok and any("non-finite" in r for r in m["reasons"])


def test_lse_finite_where_selection_is_empty_fails():
    o, l = ref()
    lg = l.copy()
    lg[2, 3] = 7.0
    ok, m = check(o.copy(), lg, o, l)
    assert not ok and any("-inf" in r for r in m["reasons"])


def test_nonzero_o_where_selection_is_empty_fails():
    o, l = ref()
    og = o.copy()
    og[2, 3, 511] = 1e-30  # any nonzero value, however small
    ok, m = check(og, l.copy(), o, l)
    assert not ok and any("O must be 0" in r for r in m["reasons"])


@pytest.mark.parametrize("f,passes", [(0.99, True), (1.01, False)])
def test_max_abs_threshold(f, passes):
    o, l = ref()
    og = o.copy()
    og[0, 2, 17] += f * MAX_ABS  # one element; rel-L2 stays tiny
    ok, m = check(og, l.copy(), o, l)
    assert m["rel_l2"] < REL_L2 / 10
    assert ok == passes, m
    assert m["max_abs"] == pytest.approx(f * MAX_ABS, rel=1e-9)


@pytest.mark.parametrize("f,passes", [(0.99, True), (1.01, False)])
def test_rel_l2_threshold(f, passes):
    # O_ref = 1 everywhere (n elements, norm sqrt(n)); adding d to every
    # element gives rel-L2 = d exactly, with max-abs d far below its bound
    n = T * H * DV
    o = np.ones((T, H, DV))
    l = np.full((T, H), 6.0)
    d = f * REL_L2
    ok, m = check(o + d, l.copy(), o, l)
    assert m["rel_l2"] == pytest.approx(d, rel=1e-9)
    assert m["max_abs"] < MAX_ABS
    assert ok == passes, m
    # one element off by e: rel-L2 = e / sqrt(n) (the normaliser is the
    # reference's norm, not the element count or the GPU's norm)
    og = o.copy()
    og[1, 1, 1] += 0.5
    assert check(og, l, o, l)[1]["rel_l2"] == pytest.approx(0.5 / np.sqrt(n), rel=1e-9)


def test_rel_l2_is_scale_invariant_and_normalised_by_the_reference():
    o, l = ref()
    og = o + 1e-3
    r1 = check(og, l, o, l)[1]["rel_l2"]
    r2 = check(4.0 * og, l, 4.0 * o, l)[1]["rel_l2"]
    assert r1 == pytest.approx(r2, rel=1e-12)
    # swapping the roles changes the normaliser: ||o+e|| != ||o||
    r3 = check(o, l, og, l)[1]["rel_l2"]
    assert r3 != pytest.approx(r1, rel=1e-12)


@pytest.mark.parametrize("f,passes", [(0.99, True), (1.01, False)])
def test_lse_threshold(f, passes):
    o, l = ref()
    lg = l.copy()
    lg[1, 0] -= f * LSE_ABS
    ok, m = check(o.copy(), lg, o, l)
    assert ok == passes, m
    assert m["lse_max_abs"] == pytest.approx(f * LSE_ABS, rel=1e-9)


def test_all_empty_passes_only_with_zero_output():
    o = np.zeros((T, H, DV))
    l = np.full((T, H), -np.inf)
    assert check(o.copy(), l.copy(), o, l)[0]
    og = o.copy()
    og[0, 0, 0] = -0.0  # negative zero equals zero
    assert check(og, l.copy(), o, l)[0]
    og[0, 0, 1] = 1e-3
    assert not check(og, l.copy(), o, l)[0]


def test_shape_mismatch_is_an_error():
    o, l = ref()
    with pytest.raises(AssertionError):
        check(o[:, :2], l, o, l)


def test_bar_no_looser_than_pages():
    # The pages report their split-K MMA kernel agreeing with the per-head
    # SIMT kernel to a relative error of at most 6.7e-3 (page "The Moment of
    # Truth: Validating Split-K Parallelization for Blackwell MLA Decode",
    # section "The Results Unfold in Real Time"); the relative bar here must
    # not be looser than that.
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))
    assert REL_L2 <= g["tolerance_context"]["value"]
    # and an error of the pages' size is rejected by the bar
    o, lse = ref()
    rng = np.random.default_rng(3)
    d = rng.normal(0.0, 1.0, o.shape)
    d[2, 3] = 0.0
    d *= g["tolerance_context"]["value"] * np.linalg.norm(o) / np.linalg.norm(d)
    ok, m = check(o + d, lse, o, lse, max_abs=np.inf)
    assert not ok and abs(m["rel_l2"] - g["tolerance_context"]["value"]) < 1e-9

"""Pins of the parity metrics every GPU verdict is judged by (oracle/moe.py:
rel_l2, max_abs_ratio).

The bars are relative L2 ||got - ref||_2 / ||ref||_2 over the whole output
tensor and max |got - ref| <= c * max |ref|.  The cases below are built so that
each plausible slip changes the result:
  * the norm of `got` in the denominator instead of `ref`'s;
  * a dropped absolute value in either maximum (negative extremes);
  * a per-row mean instead of one norm over the whole tensor;
  * a squared (not square-rooted) norm.
Values are worked out by hand as exact fractions and square roots.
"""
import math

import numpy as np
import pytest
import torch

from oracle.moe import max_abs_ratio, rel_l2


def test_rel_l2_hand_values():
    got = np.array([1.0, 2.0, 3.0])
    ref = np.array([1.0, 2.0, 5.0])
    # diff (0, 0, -2): |diff| = 2; |ref| = sqrt(1 + 4 + 25) = sqrt(30)
    assert rel_l2(got, ref) == pytest.approx(2.0 / math.sqrt(30.0), rel=1e-15)
    # the denominator is ref's norm: swapping the arguments gives 2 / sqrt(14)
    assert rel_l2(ref, got) == pytest.approx(2.0 / math.sqrt(14.0), rel=1e-15)
    assert rel_l2(got, ref) != pytest.approx(rel_l2(ref, got))


def test_rel_l2_is_one_norm_over_the_whole_tensor():
    got = np.array([[3.0, 0.0], [0.0, 10.0]])
    ref = np.array([[4.0, 0.0], [0.0, 10.0]])
    # whole tensor: |diff| = 1, |ref| = sqrt(116)
    assert rel_l2(got, ref) == pytest.approx(1.0 / math.sqrt(116.0), rel=1e-15)
    # a mean of per-row ratios would be (1/4 + 0) / 2 = 0.125
    assert rel_l2(got, ref) != pytest.approx(0.125)
    # not the squared ratio 1/116
    assert rel_l2(got, ref) != pytest.approx(1.0 / 116.0)


def test_max_abs_ratio_hand_values():
    # the largest deviation is negative: without the abs the numerator would be 1
    got = np.array([0.0, -2.0, 5.0])
    ref = np.array([0.0, 2.0, 4.0])
    # diff (0, -4, 1): max |diff| = 4; max |ref| = 4
    assert max_abs_ratio(got, ref) == pytest.approx(1.0, rel=1e-15)
    # the largest reference magnitude is negative: without the abs the
    # denominator would be 1
    got2 = np.array([-6.0, 1.0, 0.5])
    ref2 = np.array([-8.0, 1.0, 0.0])
    # diff (2, 0, 0.5): max |diff| = 2; max |ref| = 8
    assert max_abs_ratio(got2, ref2) == pytest.approx(0.25, rel=1e-15)
    # the denominator is ref's maximum, not got's (max |got2| = 6)
    assert max_abs_ratio(ref2, got2) == pytest.approx(2.0 / 6.0, rel=1e-15)


def test_metrics_zero_for_equal_tensors_and_scale_free():
    rng = np.random.default_rng(7)
    ref = rng.standard_normal((5, 9))
    assert rel_l2(ref, ref) == 0.0 and max_abs_ratio(ref, ref) == 0.0
    got = ref + 1e-3 * rng.standard_normal((5, 9))
    for s in (2.0 ** -20, 3.0, 2.0 ** 30):        # both metrics are relative
        assert rel_l2(s * got, s * ref) == pytest.approx(rel_l2(got, ref), rel=1e-12)
        assert max_abs_ratio(s * got, s * ref) == pytest.approx(max_abs_ratio(got, ref), rel=1e-12)


def test_metrics_against_torch_float64():
    # a library routine, independent of the oracle's numpy code
    rng = np.random.default_rng(11)
    ref = rng.standard_normal((7, 13)) * 3.0
    got = ref + rng.standard_normal((7, 13)) * 0.01
    tg, tr = torch.from_numpy(got), torch.from_numpy(ref)
    want_rel = (torch.linalg.vector_norm(tg - tr) / torch.linalg.vector_norm(tr)).item()
    want_max = ((tg - tr).abs().max() / tr.abs().max()).item()
    assert rel_l2(got, ref) == pytest.approx(want_rel, rel=1e-14)
    assert max_abs_ratio(got, ref) == pytest.approx(want_max, rel=1e-14)


def test_metrics_accept_low_precision_inputs():
    # BF16 outputs arrive as float32 arrays: the metrics promote to float64
    got = np.array([1.0, 2.0, 3.0], dtype=np.float32)
    ref = np.array([1.0, 2.0, 5.0], dtype=np.float64)
    assert rel_l2(got, ref) == pytest.approx(2.0 / math.sqrt(30.0), rel=1e-15)

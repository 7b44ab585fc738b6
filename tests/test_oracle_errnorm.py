"""Pins of the comparison every parity assertion goes through:
normwise relative error max_i |g_i - o_i| / max_i |o_i| (the reading of
"max relative error" for outputs that contain zeros).  Hand-computed values
chosen so that a wrong denominator (max |got|), a mean in place of a max, a
missing absolute value or a NaN that slips through each fail a case."""

import numpy as np

import oracle


def test_hand_values():
    # |diff| max 1 at the last element, max |ref| 4: 1/4 (max |got| would give 1/3)
    assert oracle.normwise_rel_err([1.0, 2.0, 3.0], [1.0, 2.0, 4.0]) == 0.25
    # largest |ref| is a negative entry: 1/8 (no absolute value would give 1/1)
    assert oracle.normwise_rel_err([-7.0, 1.0], [-8.0, 1.0]) == 0.125
    # one large difference among zeros: the max, not the mean (0.5/2 vs 0.5/6)
    assert oracle.normwise_rel_err([0.0, 2.5, 0.0], [0.0, 2.0, 0.0]) == 0.25
    # a negative difference counts by its magnitude
    assert oracle.normwise_rel_err([1.0, -3.0], [1.0, -2.0]) == 0.5
    # identical arrays, any shape
    a = np.arange(12, dtype=np.float16).reshape(3, 4)
    assert oracle.normwise_rel_err(a, a) == 0.0


def test_fp16_inputs_are_compared_exactly_in_float64():
    # 2049 is not an fp16 value; the inputs here are fp16 2048 and 2050
    g = np.array([2050.0], dtype=np.float16)
    r = np.array([2048.0], dtype=np.float16)
    assert oracle.normwise_rel_err(g, r) == 2.0 / 2048.0


def test_zero_reference():
    assert oracle.normwise_rel_err(np.zeros(5), np.zeros(5)) == 0.0
    assert oracle.normwise_rel_err([0.0, 1e-30], [0.0, 0.0]) == np.inf


def test_nan_or_inf_in_got_never_passes():
    for bad in (np.nan, np.inf, -np.inf):
        e = oracle.normwise_rel_err([1.0, bad], [1.0, 2.0])
        assert not (e <= 2e-2)
        e0 = oracle.normwise_rel_err([0.0, bad], [0.0, 0.0])
        assert not (e0 <= 2e-2)


def test_empty_arrays():
    assert oracle.normwise_rel_err(np.zeros(0), np.zeros(0)) == 0.0

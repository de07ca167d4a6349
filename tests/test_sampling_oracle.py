"""Pins of the fused-sampling oracle (``oracle/sampling.py``): closed forms
of the softmax, the nucleus and the inverse-CDF draw."""
import math

import numpy as np

from oracle import sampling


def test_values_of_decodes_both_dtypes():
    f = np.array([1.5, -2.0, np.inf], dtype=np.float32)
    assert np.array_equal(sampling.values_of(f.view(np.uint32)), f.astype(np.float64))
    bf = np.array([0x3FC0, 0xC000, 0xFF80], dtype=np.uint16)  # 1.5, -2, -inf
    assert sampling.values_of(bf).tolist() == [1.5, -2.0, -np.inf]


def test_softmax_closed_forms():
    # equal values: uniform
    assert np.allclose(sampling.softmax(np.full(7, 3.25)), np.full(7, 1 / 7), rtol=0, atol=1e-15)
    # two values d apart at temperature t: the logistic of d / t
    for d, t in [(1.0, 1.0), (2.5, 0.5), (0.1, 3.0)]:
        p = sampling.softmax(np.array([d, 0.0]), t)
        assert math.isclose(p[0], 1 / (1 + math.exp(-d / t)), rel_tol=1e-14)
        assert math.isclose(p.sum(), 1.0, rel_tol=1e-15)
    # shift invariance, and -inf / NaN entries weigh nothing
    v = np.array([4.0, 1.0, -3.0])
    assert np.allclose(sampling.softmax(v), sampling.softmax(v + 100.0), rtol=1e-13)
    p = sampling.softmax(np.array([2.0, 1.0, -np.inf, np.nan]))
    assert p[2] == 0.0 and p[3] == 0.0 and math.isclose(p[0], 1 / (1 + math.exp(-1.0)), rel_tol=1e-14)
    # a row with nothing finite
    assert sampling.softmax(np.array([-np.inf, -np.inf])).tolist() == [0.0, 0.0]
    assert sampling.softmax(np.array([np.nan, 1.0])).tolist() == [0.0, 0.0]


def test_softmax_infinite_maximum_is_the_limit():
    # the softmax of [M, M, 5, 1] as M grows tends to [1/2, 1/2, 0, 0]; the
    # definition takes that limit when M is +inf
    big = sampling.softmax(np.array([700.0, 700.0, 5.0, 1.0]))
    assert np.allclose(big, [0.5, 0.5, 0.0, 0.0], atol=1e-300)
    assert sampling.softmax(np.array([np.inf, np.inf, 5.0, 1.0, -np.inf])).tolist() == [0.5, 0.5, 0, 0, 0]
    assert sampling.softmax(np.array([np.inf, 3.0]), 0.5).tolist() == [1.0, 0.0]
    p = sampling.softmax(np.array([np.inf, np.inf, np.inf, 2.0]))
    assert [sampling.sample_position(p, 1.0, u) for u in (0.0, 0.34, 0.67, 0.99)] == [0, 1, 2, 2]


def test_nucleus_and_draw():
    p = np.array([0.5, 0.25, 0.125, 0.125])
    assert sampling.nucleus_end(p, 1.0) == 3
    assert sampling.nucleus_end(p, 0.5) == 0
    assert sampling.nucleus_end(p, 0.6) == 1
    assert sampling.nucleus_end(p, 0.875) == 2
    # inverse CDF over the whole row: cumulative 0.5, 0.75, 0.875, 1
    assert [sampling.sample_position(p, 1.0, u) for u in (0.0, 0.49, 0.5, 0.74, 0.8, 0.9, 0.999)] == \
        [0, 0, 1, 1, 2, 3, 3]
    # inside the nucleus {0, 1} (probability 0.75): thresholds at 0.5/0.75
    assert [sampling.sample_position(p, 0.6, u) for u in (0.0, 0.66, 0.67, 0.999)] == [0, 0, 1, 1]
    # top_p at or below the first probability always draws position 0
    assert all(sampling.sample_position(p, 0.3, u) == 0 for u in np.linspace(0, 0.999, 11))
    assert sampling.sample_position(np.zeros(3), 1.0, 0.5) == -1


def test_draw_frequencies_follow_the_probabilities():
    # u on a fine uniform grid reproduces the probabilities as frequencies
    p = sampling.softmax(np.array([3.0, 2.0, 2.0, 0.5, -1.0]), 0.8)
    us = (np.arange(20000) + 0.5) / 20000
    counts = np.bincount([sampling.sample_position(p, 1.0, u) for u in us], minlength=len(p))
    assert np.allclose(counts / len(us), p, atol=1e-4)

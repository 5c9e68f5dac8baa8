"""Pins of the oracle's token selection (softmax at temperature T over the k
selected values, top-p nucleus, inverse-CDF draw from the caller's uniform),
by hand-computed cases and by the draw's distribution over a grid of u."""
import math

import numpy as np
import pytest

import oracle

IDX = np.array([101, 202, 303, 404, 505, 606, 707, 808, 909, 1010], dtype=np.int32)


def test_single_pair_is_always_drawn():
    for u in (0.0, 0.5, 0.999):
        for p in (0.01, 1.0):
            tok, n, _ = oracle.sample_topp([3.5], [42], 1.0, p, u)
            assert (tok, n) == (42, 1)


def test_two_way_by_hand():
    # weights 1 and 1/3: probabilities 3/4 and 1/4
    z = [math.log(3.0), 0.0]
    assert oracle.sample_topp(z, IDX[:2], 1.0, 1.0, 0.70)[:2] == (101, 2)
    assert oracle.sample_topp(z, IDX[:2], 1.0, 1.0, 0.80)[:2] == (202, 2)
    # nucleus: 3/4 already reaches 0.7, so only the first pair can be drawn
    assert oracle.sample_topp(z, IDX[:2], 1.0, 0.70, 0.99)[:2] == (101, 1)
    assert oracle.sample_topp(z, IDX[:2], 1.0, 0.76, 0.99)[:2] == (202, 2)


def test_temperature_by_hand():
    # T = 2: weights 1 and 3^-1/2, p0 = 1 / (1 + 0.57735) = 0.63397
    z = [math.log(3.0), 0.0]
    assert oracle.sample_topp(z, IDX[:2], 2.0, 1.0, 0.63)[0] == 101
    assert oracle.sample_topp(z, IDX[:2], 2.0, 1.0, 0.64)[0] == 202
    _, _, cum = oracle.sample_topp(z, IDX[:2], 2.0, 1.0, 0.5)
    assert cum[1] == pytest.approx(1.0 + 3.0 ** -0.5, rel=1e-15)


def test_three_way_nucleus_by_hand():
    # weights 1, 1/2, 1/4 (sum 1.75); top_p = 0.8 -> the prefix 1.5 >= 1.4: n = 2
    z = [0.0, -math.log(2.0), -math.log(4.0)]
    tok, n, cum = oracle.sample_topp(z, IDX[:3], 1.0, 0.8, 0.5)
    assert (tok, n) == (101, 2)
    assert np.allclose(cum, [1.0, 1.5, 1.75])
    assert oracle.sample_topp(z, IDX[:3], 1.0, 0.8, 0.7)[:2] == (202, 2)   # 0.7 * 1.5 = 1.05 > 1
    assert oracle.sample_topp(z, IDX[:3], 1.0, 1.0, 0.9)[:2] == (303, 3)   # 0.9 * 1.75 = 1.575 > 1.5


def test_flat_weights_draw_uniformly():
    z = np.full(10, 2.25)
    for u in (0.05, 0.15, 0.55, 0.95):
        assert oracle.sample_topp(z, IDX, 1.0, 1.0, u)[0] == IDX[int(u * 10)]


def test_nan_weighs_zero_and_an_all_nan_row_takes_the_first_pair():
    z = [1.0, float("nan"), 0.5]
    tok, n, cum = oracle.sample_topp(z, IDX[:3], 1.0, 1.0, 0.999)
    assert tok == 303 and n == 3 and cum[1] == cum[0]
    assert oracle.sample_topp([float("nan")] * 3, IDX[:3], 1.0, 0.5, 0.7)[:2] == (101, 1)


def test_draw_frequencies_match_the_nucleus_distribution():
    rng = np.random.default_rng(5)
    z = np.sort(rng.normal(0.0, 2.0, 10))[::-1]
    T, p = 1.3, 0.9
    w = np.exp((z - z[0]) / T)
    c = np.cumsum(w)
    n = int(np.argmax(c >= p * c[-1])) + 1
    probs = w[:n] / c[n - 1]
    grid = 20000
    counts = np.zeros(n)
    for i in range(grid):
        tok, nn, _ = oracle.sample_topp(z, IDX, T, p, (i + 0.5) / grid)
        assert nn == n
        counts[list(IDX).index(tok)] += 1
    assert np.allclose(counts / grid, probs, atol=2.0 / grid)

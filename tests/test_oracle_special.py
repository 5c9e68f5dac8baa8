"""Pins of the oracle's top-k selection, GELU and soft-cap."""
import math

import numpy as np
import pytest

import oracle


def brute_topk(y, k):
    """Selection by Python's sort with an explicit key: numbers before NaN,
    then larger value first, then lower index first."""
    key = lambda i: (math.isnan(y[i]), 0.0 if math.isnan(y[i]) else -y[i], i)
    return sorted(range(len(y)), key=key)[:k]


@pytest.mark.parametrize("n,k", [(1, 1), (10, 10), (1000, 1), (1000, 10), (5000, 64)])
def test_topk_random(n, k):
    y = np.random.default_rng(n + k).standard_normal(n)
    assert oracle.topk(y, k).tolist() == brute_topk(y.tolist(), k)


def test_topk_ties_prefer_lower_index():
    y = np.array([1.0, 3.0, 3.0, 2.0, 3.0, -0.0, 0.0])
    assert oracle.topk(y, 4).tolist() == [1, 2, 4, 3]
    # -0.0 and +0.0 compare equal: lower index first
    assert oracle.topk(np.array([-0.0, 0.0]), 2).tolist() == [0, 1]
    assert oracle.topk(np.array([0.0, -0.0]), 2).tolist() == [0, 1]


def test_topk_nan_last_and_infinities():
    y = np.array([np.nan, -np.inf, 1.0, np.nan, np.inf, -5.0])
    assert oracle.topk(y, 6).tolist() == [4, 2, 5, 1, 0, 3]
    assert oracle.topk(y, 6).tolist() == brute_topk(y.tolist(), 6)


def test_topk_k1_is_argmax():
    y = np.random.default_rng(1).standard_normal(4097)
    assert oracle.topk(y, 1)[0] == int(np.argmax(y))


def test_topk_rejects_bad_k():
    with pytest.raises(ValueError):
        oracle.topk(np.zeros(3), 4)
    with pytest.raises(ValueError):
        oracle.topk(np.zeros(3), 0)


def test_gelu_special_values():
    g = oracle.gelu_tanh
    assert g(0.0) == 0.0
    for v in (50.0, 1e4, 1e30, 3e38):
        assert g(v) == v
        r = g(-v)
        assert r == 0.0 and not math.isnan(r)
    # odd part: gelu(v) - gelu(-v) = v
    for v in np.linspace(-6, 6, 49):
        assert abs(g(v) - g(-v) - v) <= 1e-15 * max(1.0, abs(v))


def test_gelu_close_to_erf_form():
    # the tanh form approximates v * Phi(v) to about 1e-3 absolute
    for v in np.linspace(-8, 8, 161):
        exact = 0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0)))
        assert abs(oracle.gelu_tanh(v) - exact) < 1e-3


def test_gelu_derivative_bound_used_by_tolerance():
    v = np.linspace(-10, 10, 200001)
    gv = oracle.gelu_tanh(v)
    slope = np.abs(np.diff(gv) / np.diff(v))
    assert slope.max() < 1.13


def test_geglu_is_product():
    g = np.array([-3.0, 0.0, 0.5, 4.0])
    u = np.array([2.0, 5.0, -1.0, 0.25])
    assert np.array_equal(oracle.geglu(g, u), oracle.gelu_tanh(g) * u)


def test_softcap_properties():
    y = np.linspace(-1e6, 1e6, 20001)
    z = oracle.softcap(y, 30.0)
    assert np.all(np.abs(z) <= 30.0)
    assert np.array_equal(oracle.softcap(-y, 30.0), -z)
    assert oracle.softcap(np.array([0.0]), 30.0)[0] == 0.0
    assert np.all(np.diff(z) >= 0)
    small = np.linspace(-0.1, 0.1, 101)
    taylor = small - small**3 / (3 * 30.0**2) + 2 * small**5 / (15 * 30.0**4)
    assert np.allclose(oracle.softcap(small, 30.0), taylor, rtol=0, atol=1e-15)

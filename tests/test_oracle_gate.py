"""Pins of the oracle's reliability gate (Eq. 9-11) and token weights (Eq. 8 weights):
special cases the pages state, closed forms, and an independent library (scipy)."""
import math

import numpy as np
import pytest
from scipy import special, stats

from oracle import kvc_oracle as O


def test_identical_anchors_entropy_is_one_and_flags():
    q = np.full(7, 123.456)
    d, h, f = O.gate_decide_pages(q, tau=0.3, temp=1.0, capacity=10, n_anchors=7)
    assert h == pytest.approx(1.0, abs=1e-15)
    assert f == O.FLAG_ENTROPY


def test_distinctive_anchor_is_accepted():
    q = np.array([10.0 ** 2, 60.0 ** 2, 61.0 ** 2, 62.0 ** 2])
    d, h, f = O.gate_decide_pages(q, tau=0.3, temp=1.0, capacity=10, n_anchors=4)
    assert h < 1e-10 and f == 0


def test_single_compatible_anchor_flags():
    d, h, f = O.gate_decide_pages(np.array([4.0]), 0.3, 1.0, capacity=10, n_anchors=3)
    assert f == O.FLAG_FEW_ANCHORS


def test_empty_pool_flags():
    d, h, f = O.gate_decide_pages(np.zeros(0), 0.3, 1.0, capacity=10, n_anchors=0)
    assert f == O.FLAG_FEW_ANCHORS


def test_capacity_one_bypasses_gate():
    d, h, f = O.gate_decide_pages(np.array([4.0]), 0.3, 1.0, capacity=1, n_anchors=1)
    assert f == 0


@pytest.mark.parametrize("tau,expect", [(1.0, 0), (-0.01, O.FLAG_ENTROPY)])
def test_tau_extremes(tau, expect):
    rng = np.random.default_rng(0)
    for _ in range(20):
        q = rng.uniform(0, 50, size=rng.integers(2, 9))
        _, h, f = O.gate_decide_pages(q, tau, 1.0, capacity=20, n_anchors=q.size)
        assert 0.0 <= h <= 1.0 + 1e-15
        assert f == expect


def test_boundary_accepts_equal():
    # accept iff H <= tau ("does not exceed")
    q = np.array([1.0, 4.0])
    _, h, _ = O.gate_decide_pages(q, 0.5, 1.0, capacity=5, n_anchors=2)
    _, _, f = O.gate_decide_pages(q, h, 1.0, capacity=5, n_anchors=2)
    assert f == 0


def test_entropy_against_scipy():
    rng = np.random.default_rng(1)
    for n in (2, 3, 10, 20):
        d = rng.uniform(0, 3, size=n)
        _, h, _ = O.gate_decide_pages(d ** 2, 0.3, 1.0, capacity=n, n_anchors=n)
        g = special.softmax(-d)
        assert h == pytest.approx(stats.entropy(g, base=2) / math.log2(n), rel=1e-12)


def test_two_anchor_closed_form():
    # g = (1/(1+e^-x), e^-x/(1+e^-x)) with x = d1 - d0; H = binary entropy in bits
    d0, d1 = 1.0, 2.5
    _, h, _ = O.gate_decide_pages(np.array([d0 ** 2, d1 ** 2]), 0.3, 1.0, 2, 2)
    p = 1.0 / (1.0 + math.exp(-(d1 - d0)))
    hb = -(p * math.log2(p) + (1 - p) * math.log2(1 - p))
    assert h == pytest.approx(hb, rel=1e-13)


def test_gate_temperature_scales_distances():
    d = np.array([1.0, 2.0, 3.5])
    _, h1, _ = O.gate_decide_pages((2 * d) ** 2, 0.3, 2.0, 3, 3)
    _, h2, _ = O.gate_decide_pages(d ** 2, 0.3, 1.0, 3, 3)
    assert h1 == pytest.approx(h2, rel=1e-14)


def test_weights_rows_sum_to_one_and_match_scipy():
    rng = np.random.default_rng(2)
    m = rng.uniform(0.5, 1.5, size=(50, 20))
    w = O.token_weights(m, 0.1, O.PAGES)
    assert np.max(np.abs(w.sum(axis=1) - 1)) < 1e-15
    assert np.allclose(w, special.softmax(-m / 0.1, axis=1), rtol=1e-13, atol=0)
    c = rng.uniform(-1, 1, size=(50, 20))
    assert np.allclose(O.token_weights(c, 0.1, O.COS_R), special.softmax(c / 0.1, axis=1), rtol=1e-13)


def test_weights_permutation_equivariant():
    rng = np.random.default_rng(3)
    m = rng.uniform(size=(10, 6))
    perm = rng.permutation(6)
    assert np.allclose(O.token_weights(m[:, perm], 0.7, O.PAGES), O.token_weights(m, 0.7, O.PAGES)[:, perm],
                       rtol=0, atol=1e-16)


def test_weights_temperature_limits():
    rng = np.random.default_rng(4)
    m = rng.uniform(size=(10, 6))
    w0 = O.token_weights(m, 1e-6, O.PAGES)
    assert np.array_equal(np.argmax(w0, axis=1), np.argmin(m, axis=1))
    assert np.allclose(w0.max(axis=1), 1.0, atol=1e-12)
    winf = O.token_weights(m, 1e9, O.PAGES)
    assert np.allclose(winf, 1.0 / 6, atol=1e-9)


def test_cosine_gate_flags():
    pa = np.array([9.0, 1.0])
    pp = np.array([9.0, 4.0])
    aa = np.array([9.0, 4.0])
    c, best, f = O.gate_decide_cos(pa, pp, aa, 0.5, capacity=5, n_anchors=2)
    assert c[0] == pytest.approx(1.0) and c[1] == pytest.approx(0.25)
    assert best == pytest.approx(1.0) and f == 0
    _, _, f = O.gate_decide_cos(pa, pp, aa, 1.5, capacity=5, n_anchors=2)
    assert f == O.FLAG_COS_BELOW
    _, _, f = O.gate_decide_cos(pa, pp, aa, 1.5, capacity=1, n_anchors=1)
    assert f == 0

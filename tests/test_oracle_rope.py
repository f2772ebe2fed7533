"""Pins of the oracle's key re-alignment (rotate-half RoPE) against closed forms and
the group/relative-position invariants that any rotary encoding must satisfy."""
import math

import numpy as np
import pytest

from oracle import kvc_oracle as O


def test_frequency_closed_form():
    # w_c = theta^(-2c/d_h): w_0 = 1 and, for d_h = 128, w_32 = 10000^(-1/2) = 0.01 exactly
    w = O.inv_freq(128, 10000.0)
    assert w[0] == 1.0
    assert abs(w[32] - 0.01) < 1e-17
    assert abs(w[16] - 0.1) < 1e-16
    assert np.all(np.diff(w) < 0)


def test_zero_shift_is_bit_exact_identity():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 5, 256))
    y = O.rope(x, 0, 128)
    assert np.array_equal(x, y)


def test_one_hot_pairing_and_sign():
    # channel c pairs with c + d_h/2 and turns counter-clockwise by p * w_c
    d_h, p = 8, 3
    w = O.inv_freq(d_h)
    for c in range(d_h // 2):
        e = np.zeros(2 * d_h)
        e[d_h + c] = 1.0                       # second head, first half
        y = O.rope(e, p, d_h)
        nz = np.flatnonzero(np.abs(y) > 0)
        assert set(nz) <= {d_h + c, d_h + c + d_h // 2}
        assert y[d_h + c] == pytest.approx(math.cos(p * w[c]), abs=1e-15)
        assert y[d_h + c + d_h // 2] == pytest.approx(math.sin(p * w[c]), abs=1e-15)
        e2 = np.zeros(2 * d_h)
        e2[c + d_h // 2] = 1.0                 # first head, second half
        y2 = O.rope(e2, p, d_h)
        assert y2[c] == pytest.approx(-math.sin(p * w[c]), abs=1e-15)
        assert y2[c + d_h // 2] == pytest.approx(math.cos(p * w[c]), abs=1e-15)


def test_worked_example_head_dim_4():
    # d_h = 4: pairs (0,2) at w=1 and (1,3) at w=0.01; x = (1,2,3,4), shift 1
    y = O.rope(np.array([1.0, 2.0, 3.0, 4.0]), 1, 4)
    c1, s1 = math.cos(1.0), math.sin(1.0)
    c2, s2 = math.cos(0.01), math.sin(0.01)
    exp = [1 * c1 - 3 * s1, 2 * c2 - 4 * s2, 1 * s1 + 3 * c1, 2 * s2 + 4 * c2]
    assert np.allclose(y, exp, rtol=0, atol=1e-15)


@pytest.mark.parametrize("a,b", [(5, 7), (-300, 812), (1, -1), (32768, 17)])
def test_group_property(a, b):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 256))
    lhs = O.rope(O.rope(x, a, 128), b, 128)
    rhs = O.rope(x, a + b, 128)
    # fp64 angle rounding grows with |position|: allow a few ulps of the largest angle
    tol = 8 * 2.0 ** -53 * (abs(a) + abs(b) + 1) * np.max(np.abs(x))
    assert np.max(np.abs(lhs - rhs)) <= tol


def test_shift_equals_direct_position():
    # R(s) applied to a key encoded at p equals the key encoded at p + s
    rng = np.random.default_rng(2)
    k = rng.standard_normal((6, 1024))
    p, s = 512, 300
    tol = 8 * 2.0 ** -53 * (p + s + 1) * np.max(np.abs(k))
    assert np.max(np.abs(O.rope(O.rope(k, p, 128), s, 128) - O.rope(k, p + s, 128))) <= tol


def test_norm_per_pair_preserved():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 256))
    y = O.rope(x, 12345, 64)
    xh = x.reshape(5, 4, 64)
    yh = y.reshape(5, 4, 64)
    nx = xh[..., :32] ** 2 + xh[..., 32:] ** 2
    ny = yh[..., :32] ** 2 + yh[..., 32:] ** 2
    assert np.max(np.abs(nx - ny)) < 1e-13


def test_relative_position_property():
    # <R(m) q, R(n) k> depends on m - n only
    rng = np.random.default_rng(4)
    q = rng.standard_normal(128)
    k = rng.standard_normal(128)
    v1 = O.rope(q, 1000, 128) @ O.rope(k, 900, 128)
    v2 = O.rope(q, 100, 128) @ O.rope(k, 0, 128)
    assert abs(v1 - v2) < 1e-11


def test_inverse_shift():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 128))
    y = O.rope(O.rope(x, 777, 128), -777, 128)
    assert np.max(np.abs(y - x)) < 1e-13

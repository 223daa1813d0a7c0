"""Pins of the oracle's RoPE (rotary position embedding on the QKV product's output).

The pages name RoPE among the element-wise transforms the reparameterisation covers
(kucoin page, sections "CODA: El epilogo esconde un tesoro" and "Cinco bloques y un
lenguaje LEGO") without defining it; the LLaMA definition is used: in each head of 64
values, value i pairs with value i + 32 and the pair turns by pos * base^(-2i/64).
Each pin below checks that definition by a route that does not retype the oracle's
formula: the complex-exponential form (numpy complex128), the rotation group laws, the
relative-position property, and the pass-through of the V columns.
"""

import numpy as np
import pytest

import oracle

BASE = 500000.0
HD = 64


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _complex_rope(y, pos, base, head_dim, rot_cols):
    # x1 + i x2 times exp(i pos theta_j), head by head, with numpy's complex arithmetic
    out = y.copy()
    half = head_dim // 2
    j = np.arange(half)
    theta = np.power(base, -2.0 * j / head_dim)
    for h0 in range(0, rot_cols, head_dim):
        z = y[:, h0:h0 + half] + 1j * y[:, h0 + half:h0 + head_dim]
        z = z * np.exp(1j * np.outer(pos, theta))
        out[:, h0:h0 + half] = z.real
        out[:, h0 + half:h0 + head_dim] = z.imag
    return out


def test_position_zero_is_identity():
    y = _rand((4, 3 * HD), 1)
    assert np.array_equal(oracle.rope(y, [0] * 4, BASE, HD, 2 * HD), y)


def test_v_columns_pass_through():
    y = _rand((5, 5 * HD), 2)
    o = oracle.rope(y, [0, 1, 77, 4095, 12345], BASE, HD, 3 * HD)
    assert np.array_equal(o[:, 3 * HD:], y[:, 3 * HD:])
    assert not np.allclose(o[1:, :3 * HD], y[1:, :3 * HD])


def test_matches_complex_exponential_form():
    y = _rand((6, 4 * HD), 3)
    pos = np.array([1, 2, 3, 100, 2047, 4095])
    o = oracle.rope(y, pos, BASE, HD, 3 * HD)
    ref = _complex_rope(y, pos, BASE, HD, 3 * HD)
    assert np.allclose(o, ref, rtol=0, atol=1e-12)


def test_pair_norms_are_preserved():
    y = _rand((8, 2 * HD), 4)
    pos = np.arange(8) * 513
    o = oracle.rope(y, pos, BASE, HD, 2 * HD)
    for h0 in (0, HD):
        n_in = y[:, h0:h0 + 32] ** 2 + y[:, h0 + 32:h0 + HD] ** 2
        n_out = o[:, h0:h0 + 32] ** 2 + o[:, h0 + 32:h0 + HD] ** 2
        assert np.allclose(n_out, n_in, rtol=1e-12, atol=0)


def test_rotations_compose():
    # turning by p1 then by p2 is turning by p1 + p2
    y = _rand((3, HD), 5)
    p1 = np.array([7, 300, 1000])
    p2 = np.array([11, 5, 2000])
    two = oracle.rope(oracle.rope(y, p1, BASE, HD, HD), p2, BASE, HD, HD)
    one = oracle.rope(y, p1 + p2, BASE, HD, HD)
    assert np.allclose(two, one, rtol=0, atol=1e-11)


def test_relative_position_property():
    # <rope(q, a), rope(k, b)> depends only on a - b
    q, k = _rand((1, HD), 6), _rand((1, HD), 7)
    a, b = 1234, 1200
    dots = []
    for shift in (0, 1, 17, 2000):
        rq = oracle.rope(q, [a + shift], BASE, HD, HD)
        rk = oracle.rope(k, [b + shift], BASE, HD, HD)
        dots.append(float((rq @ rk.T)[0, 0]))
    assert np.allclose(dots, dots[0], rtol=1e-11, atol=1e-12)


def test_layout_errors_are_rejected():
    y = _rand((2, 3 * HD), 8)
    with pytest.raises(ValueError):
        oracle.rope(y, [0, 1], BASE, HD, HD + 1)      # rot_cols not whole heads
    with pytest.raises(ValueError):
        oracle.rope(y, [0, 1], BASE, HD, 4 * HD)      # beyond the columns
    with pytest.raises(ValueError):
        oracle.rope(y, [0], BASE, HD, HD)             # one position per row

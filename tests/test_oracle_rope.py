"""Pins of the oracle's inverse RoPE ("DSV4 Audit", A4: the attention output
is rotated back by RoPE(-pos) at the query position).

The pins come from outside the oracle's own formula: the identity at
position 0, the library sine and cosine for the unit-frequency pair, the
geometric frequency schedule read back from the rotation angles, composition
with a forward rotation written as complex multiplication, the group law of
rotations, and the relative-position property that makes the de-rotation
useful.
"""
import math

import numpy as np
import pytest

import oracle

D_NOPE, D_ROPE = 448, 64
THETA = 10000.0


def rand_rows(seed, n=3, d=D_NOPE + D_ROPE):
    return np.random.default_rng(seed).standard_normal((n, d))


def test_position_zero_is_identity():
    o = rand_rows(1)
    assert np.array_equal(oracle.inverse_rope(o, 0, D_NOPE, THETA), o)


def test_nope_dims_untouched():
    o = rand_rows(2)
    r = oracle.inverse_rope(o, 12345, D_NOPE, THETA)
    assert np.array_equal(r[:, :D_NOPE], o[:, :D_NOPE])


@pytest.mark.parametrize("pos", [1, 7, 255, 524287])
def test_unit_frequency_pair_against_library_sin_cos(pos):
    # pair 0 turns at frequency theta^0 = 1: e_0 goes to (cos p, -sin p) and
    # e_1 to (sin p, cos p) under the rotation by -p
    o = np.zeros((2, D_NOPE + D_ROPE))
    o[0, D_NOPE] = 1.0
    o[1, D_NOPE + 1] = 1.0
    r = oracle.inverse_rope(o, pos, D_NOPE, THETA)
    assert r[0, D_NOPE] == pytest.approx(math.cos(pos), abs=1e-12)
    assert r[0, D_NOPE + 1] == pytest.approx(-math.sin(pos), abs=1e-12)
    assert r[1, D_NOPE] == pytest.approx(math.sin(pos), abs=1e-12)
    assert r[1, D_NOPE + 1] == pytest.approx(math.cos(pos), abs=1e-12)
    # no other dim moves
    mask = np.ones(D_NOPE + D_ROPE, bool)
    mask[D_NOPE:D_NOPE + 2] = False
    assert not r[:, mask].any()


@pytest.mark.parametrize("d_nope,d_rope,theta", [(448, 64, 10000.0), (48, 16, 10000.0), (448, 64, 1e6)])
def test_frequencies_form_the_rotary_geometric_schedule(d_nope, d_rope, theta):
    # rotate the first unit vector of every pair by one position and read the
    # angle back: it is -f_i with f_0 = 1, f_{i+1} / f_i = theta^(-2/d_rope)
    o = np.zeros((d_rope // 2, d_nope + d_rope))
    for i in range(d_rope // 2):
        o[i, d_nope + 2 * i] = 1.0
    r = oracle.inverse_rope(o, 1, d_nope, theta)
    f = np.array([-math.atan2(r[i, d_nope + 2 * i + 1], r[i, d_nope + 2 * i]) for i in range(d_rope // 2)])
    assert f[0] == pytest.approx(1.0, rel=1e-14)
    assert np.allclose(f[1:] / f[:-1], theta ** (-2.0 / d_rope), rtol=1e-12)
    assert f[-1] == pytest.approx(theta ** (-(d_rope - 2) / d_rope), rel=1e-12)


def forward_rope_complex(o, pos, d_nope, theta):
    # forward rotary embedding as complex multiplication: pair i of the rope
    # part is the complex number (x, y), multiplied by exp(1j * pos * f_i)
    z = o[..., d_nope::2] + 1j * o[..., d_nope + 1::2]
    d_rope = o.shape[-1] - d_nope
    f = np.array([theta ** (-(2.0 * i) / d_rope) for i in range(d_rope // 2)])
    z = z * np.exp(1j * pos * f)
    out = o.copy()
    out[..., d_nope::2] = z.real
    out[..., d_nope + 1::2] = z.imag
    return out


@pytest.mark.parametrize("pos", [3, 8191, 524287])
def test_inverse_undoes_forward_rotation(pos):
    o = rand_rows(3)
    back = oracle.inverse_rope(forward_rope_complex(o, pos, D_NOPE, THETA), pos, D_NOPE, THETA)
    assert np.allclose(back, o, atol=1e-9)


def test_group_law_and_norm():
    o = rand_rows(4)
    a = oracle.inverse_rope(oracle.inverse_rope(o, 100, D_NOPE, THETA), 23, D_NOPE, THETA)
    b = oracle.inverse_rope(o, 123, D_NOPE, THETA)
    assert np.allclose(a, b, atol=1e-12)
    # every pair keeps its length
    r = oracle.inverse_rope(o, 999, D_NOPE, THETA)
    n0 = o[:, D_NOPE::2] ** 2 + o[:, D_NOPE + 1::2] ** 2
    n1 = r[:, D_NOPE::2] ** 2 + r[:, D_NOPE + 1::2] ** 2
    assert np.allclose(n0, n1, rtol=1e-12)


def test_relative_position_property():
    # <R(-p) a, R(-q) b> == <a, R(-(q - p)) b>: after de-rotation only the
    # position difference matters
    rows = rand_rows(5, n=2)
    a, b = rows[0], rows[1]
    p, q = 1000, 1337
    lhs = oracle.inverse_rope(a, p, D_NOPE, THETA) @ oracle.inverse_rope(b, q, D_NOPE, THETA)
    rhs = a @ oracle.inverse_rope(b, q - p, D_NOPE, THETA)
    assert lhs == pytest.approx(rhs, rel=1e-10, abs=1e-10)


def test_mutant_sign_is_caught():
    # a forward rotation in place of the inverse fails the composition pin
    o = rand_rows(6)
    fwd = forward_rope_complex(o, 77, D_NOPE, THETA)
    wrong = forward_rope_complex(fwd, 77, D_NOPE, THETA)
    assert not np.allclose(wrong, o, atol=1e-3)
    assert np.allclose(oracle.inverse_rope(fwd, 77, D_NOPE, THETA), o, atol=1e-9)

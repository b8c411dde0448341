"""Pins for the oracle's real spherical harmonics (degree <= 3).

Pinned against: orthonormality on the sphere by exact quadrature, SciPy's
complex harmonics converted to the real Condon-Shortley form, the
degree-0 closed form, the familiar degree-1 signs, and central finite
differences of the gradient.
"""
import math

import numpy as np
import pytest
from scipy.special import sph_harm_y

from oracle.sh import sh_basis, sh_basis_grad, lm_of_index, num_sh


def _sphere_quadrature(n_theta=12, n_phi=16):
    # Gauss-Legendre in cos(theta) x uniform phi: exact for polynomials of
    # degree < 2 n_theta in z and trigonometric degree < n_phi in phi.
    zs, wz = np.polynomial.legendre.leggauss(n_theta)
    phis = 2 * np.pi * np.arange(n_phi) / n_phi
    Z, P = np.meshgrid(zs, phis, indexing="ij")
    W = np.outer(wz, np.full(n_phi, 2 * np.pi / n_phi))
    st = np.sqrt(1 - Z**2)
    d = np.stack([st * np.cos(P), st * np.sin(P), Z], -1).reshape(-1, 3)
    return d, W.ravel()


def test_orthonormal_to_1e12():
    d, w = _sphere_quadrature()
    Y = sh_basis(3, d)
    G = (Y * w[:, None]).T @ Y
    assert np.abs(G - np.eye(16)).max() < 1e-12


def test_matches_scipy_complex_harmonics():
    rng = np.random.default_rng(0)
    d = rng.normal(size=(200, 3))
    d /= np.linalg.norm(d, axis=1, keepdims=True)
    theta = np.arccos(np.clip(d[:, 2], -1, 1))
    phi = np.arctan2(d[:, 1], d[:, 0])
    Y = sh_basis(3, d)
    for k in range(16):
        l, m = lm_of_index(k)
        Yc = sph_harm_y(l, abs(m), theta, phi)   # includes the Condon-Shortley phase
        if m > 0:
            ref = math.sqrt(2) * Yc.real
        elif m < 0:
            ref = math.sqrt(2) * Yc.imag
        else:
            ref = Yc.real
        np.testing.assert_allclose(Y[:, k], ref, atol=1e-13, err_msg=f"l={l} m={m}")


def test_degree0_and_degree1_closed_forms():
    d = np.array([[0.36, -0.48, 0.8]])
    Y = sh_basis(1, d)[0]
    assert Y[0] == pytest.approx(1 / (2 * math.sqrt(math.pi)), abs=1e-15)
    c1 = math.sqrt(3 / (4 * math.pi))
    x, y, z = d[0]
    np.testing.assert_allclose(Y[1:], [-c1 * y, c1 * z, -c1 * x], atol=1e-15)


def test_counts():
    assert [num_sh(k) for k in range(4)] == [1, 4, 9, 16]
    assert [lm_of_index(k) for k in range(4)] == [(0, 0), (1, -1), (1, 0), (1, 1)]


def test_gradient_finite_differences():
    rng = np.random.default_rng(1)
    p = rng.normal(size=(50, 3))
    G = sh_basis_grad(3, p)
    h = 1e-6
    for j in range(3):
        e = np.zeros(3)
        e[j] = h
        fd = (sh_basis(3, p + e) - sh_basis(3, p - e)) / (2 * h)
        np.testing.assert_allclose(G[:, :, j], fd, atol=1e-8)

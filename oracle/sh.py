"""Real spherical harmonics of degree <= 3, fp64, from their definition.

Reading (the pages give no SH convention): real harmonics built from the
associated Legendre functions *with* the Condon-Shortley phase,

    m > 0:  sqrt(2) K_lm P_l^m(cos t) cos(m p)
    m < 0:  sqrt(2) K_l|m| P_l^|m|(cos t) sin(|m| p)
    m = 0:  K_l0 P_l(cos t)
    K_lm = sqrt((2l+1)/(4 pi) * (l-|m|)! / (l+|m|)!)

with t the polar angle from +z and p the azimuth from +x toward +y,
ordered l = 0..deg, m = -l..l. Colour = max(0, sum_k sh_k Y_k(d) + 0.5).

Evaluation: with P_l^m(z) = (-1)^m (1-z^2)^(m/2) d^m/dz^m P_l(z) (Rodrigues'
formula for P_l) and sin^m(t) e^{i m p} = (x + i y)^m on the unit sphere,

    Y_lm(x, y, z) = c_lm (-1)^|m| P_l^(|m|)(z) * {Re, Im}((x + i y)^|m|)

which is a polynomial in (x, y, z). Its gradient w.r.t. (x, y, z) is taken
from that polynomial; callers project it onto the sphere's tangent plane,
which removes the dependence on how the polynomial extends off the sphere.
"""
from __future__ import annotations

import math
from functools import lru_cache

import numpy as np
from numpy.polynomial import Polynomial

__all__ = ["num_sh", "sh_basis", "sh_basis_grad", "lm_of_index"]


def num_sh(degree: int) -> int:
    return (degree + 1) ** 2


def lm_of_index(k: int) -> tuple[int, int]:
    l = int(math.isqrt(k))
    return l, k - l * l - l


@lru_cache(maxsize=None)
def _legendre_deriv(l: int, m: int) -> Polynomial:
    """d^m/dz^m P_l(z), with P_l from Rodrigues' formula."""
    p = Polynomial([-1.0, 0.0, 1.0]) ** l
    p = p.deriv(l) / (2.0 ** l * math.factorial(l)) if l > 0 else Polynomial([1.0])
    return p.deriv(m) if m > 0 else p


def _norm(l: int, m: int) -> float:
    am = abs(m)
    K = math.sqrt((2 * l + 1) / (4.0 * math.pi)
                  * math.factorial(l - am) / math.factorial(l + am))
    return K * (math.sqrt(2.0) if m != 0 else 1.0)


def _xy_power(x, y, m):
    """(x + i y)^m as complex array (m >= 0)."""
    return (x + 1j * y) ** m


def sh_basis(degree: int, d: np.ndarray) -> np.ndarray:
    """Y[..., k] for unit directions d[..., 3], k = 0..(degree+1)^2-1."""
    d = np.asarray(d, np.float64)
    x, y, z = d[..., 0], d[..., 1], d[..., 2]
    out = np.empty(d.shape[:-1] + (num_sh(degree),), np.float64)
    for k in range(num_sh(degree)):
        l, m = lm_of_index(k)
        am = abs(m)
        radial = (-1.0) ** am * _legendre_deriv(l, am)(z)
        w = _xy_power(x, y, am)
        ang = w.real if m >= 0 else w.imag
        out[..., k] = _norm(l, m) * radial * ang
    return out


def sh_basis_grad(degree: int, d: np.ndarray) -> np.ndarray:
    """dY_k/d(x,y,z) of the polynomial form, shape [..., K, 3]."""
    d = np.asarray(d, np.float64)
    x, y, z = d[..., 0], d[..., 1], d[..., 2]
    out = np.zeros(d.shape[:-1] + (num_sh(degree), 3), np.float64)
    for k in range(num_sh(degree)):
        l, m = lm_of_index(k)
        am = abs(m)
        c = _norm(l, m) * (-1.0) ** am
        radial = _legendre_deriv(l, am)(z)
        radial_dz = _legendre_deriv(l, am).deriv(1)(z) if l > am else np.zeros_like(z)
        w = _xy_power(x, y, am)
        if am > 0:
            wm1 = _xy_power(x, y, am - 1)
            dw_dx = am * wm1           # d/dx (x+iy)^m
            dw_dy = 1j * am * wm1      # d/dy (x+iy)^m
        else:
            dw_dx = np.zeros_like(w)
            dw_dy = np.zeros_like(w)
        if m >= 0:
            ang, ang_dx, ang_dy = w.real, dw_dx.real, dw_dy.real
        else:
            ang, ang_dx, ang_dy = w.imag, dw_dx.imag, dw_dy.imag
        out[..., k, 0] = c * radial * ang_dx
        out[..., k, 1] = c * radial * ang_dy
        out[..., k, 2] = c * radial_dz * ang
    return out

"""Pins of the oracle's coordinate law and Lloyd-Max codebook against what the
pages and the mathematics fix (closed forms, printed values, a textbook table,
direct quadrature and Monte Carlo on the sphere). CPU only."""
import math
import os

import numpy as np
import pytest
from scipy import integrate

from oracle import (coord_density, coord_first_moment, coord_mass, coord_norm_const,
                    coord_second_moment, lloyd_max, nearest_centroid)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
D = 128


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(v) for v in line.split()])
    return rows


@pytest.fixture(scope="module")
def books():
    return {b: lloyd_max(D, b) for b in range(1, 5)}


@pytest.mark.parametrize("d", [3, 8, 128, 1000])
def test_density_normalised_and_variance(d):
    # Direct quadrature of the printed density: mass 1 and E[X²] = 1/d (the d
    # squared coordinates of a unit vector sum to 1 and share one law).
    f = lambda x: float(coord_density(x, d))
    m0 = integrate.quad(f, -1, 1, limit=200, points=[0.0])[0]
    m2 = integrate.quad(lambda x: x * x * f(x), -1, 1, limit=200, points=[0.0])[0]
    assert abs(m0 - 1) < 1e-9
    assert abs(m2 - 1 / d) < 1e-9 / d


@pytest.mark.parametrize("d", [5, 128])
def test_cell_moments_match_quadrature(d):
    g = np.random.default_rng(7)
    f = lambda x: float(coord_density(x, d))
    s = min(3 / math.sqrt(d), 0.95)
    for _ in range(6):
        a, b = np.sort(g.uniform(-s, s, 2))
        q0 = integrate.quad(f, a, b, epsabs=1e-14)[0]
        q1 = integrate.quad(lambda x: x * f(x), a, b, epsabs=1e-14)[0]
        q2 = integrate.quad(lambda x: x * x * f(x), a, b, epsabs=1e-14)[0]
        assert abs(coord_mass(a, b, d) - q0) < 1e-11
        assert abs(coord_first_moment(a, b, d) - q1) < 1e-12
        assert abs(coord_second_moment(a, b, d) - q2) < 1e-12


def test_one_bit_closed_form(books):
    # b=1 on a symmetric law: boundary 0, centroids ±E|X| = ±2 C_d/(d-1),
    # D = 1 - d (E|X|)². C_d from Γ directly.
    cd = math.gamma(D / 2) / (math.sqrt(math.pi) * math.gamma((D - 1) / 2))
    e_abs = 2 * cd / (D - 1)
    c, t, Dm = books[1]
    assert t[0] == 0.0
    np.testing.assert_allclose(c, [-e_abs, e_abs], rtol=1e-12)
    assert abs(Dm - (1 - D * e_abs ** 2)) < 1e-12
    # d → ∞: E|X|·√d → √(2/π), D → 1 - 2/π (the pages' 0.36).
    c_big, _, D_big = lloyd_max(4096, 1)
    assert abs(c_big[1] * math.sqrt(4096) - math.sqrt(2 / math.pi)) < 2e-4
    assert abs(D_big - (1 - 2 / math.pi)) < 2e-4


def test_printed_distortions(books):
    # "The Distortion Guarantee…", section "The Upper Bound": 0.36, 0.117,
    # 0.030, 0.009. The exact d=128 values are close; 0.030 is a rounding of
    # ≈0.034, hence the wider tolerance at b=3.
    tol = {1: 0.05, 2: 0.05, 3: 0.15, 4: 0.05}
    for b, printed in _golden_rows("distortion_printed.txt"):
        b = int(b)
        Dm = books[b][2]
        assert abs(Dm - printed) / printed < tol[b], (b, Dm, printed)


def test_bound_sandwich(books):
    # Lower bound 1/4^b ("The Lower Bound"); upper bound 2.72/4^b ("The Upper
    # Bound", "The Gap"), the constant read as √3·π/2 = 2.7207 because the
    # literal √(3π)/2 = 1.535 is below the pages' own printed values.
    up = math.sqrt(3) * math.pi / 2
    for b in range(1, 5):
        Dm = books[b][2]
        assert 1 / 4 ** b <= Dm <= up / 4 ** b
    # b = 1 ratio to the lower bound ≈ 1.45 ("Cái định lý đẹp" on omelet.tech).
    assert abs(books[1][2] * 4 - 1.45) < 0.02
    # The literal constant is violated at b ≥ 2 (recorded reading, not a bug).
    lit = math.sqrt(3 * math.pi) / 2
    assert all(books[b][2] > lit / 4 ** b for b in (2, 3, 4))


def test_gaussian_limit_textbook():
    # Richardson-extrapolate d → ∞ from d = 1024, 2048 and compare with the
    # textbook Lloyd-Max table for N(0,1).
    for row in _golden_rows("lloyd_max_gaussian_textbook.txt"):
        b, mse, levels = int(row[0]), row[1], np.array(row[2:])
        c1, _, D1 = lloyd_max(1024, b, tol=1e-11)
        c2, _, D2 = lloyd_max(2048, b, tol=1e-11)
        K = 1 << b
        l1 = c1[K // 2:] * math.sqrt(1024)
        l2 = c2[K // 2:] * math.sqrt(2048)
        lim = 2 * l2 - l1
        np.testing.assert_allclose(lim, levels, atol=6e-4)
        assert abs((2 * D2 - D1) - mse) / mse < 2e-3


def test_symmetry_and_sorted(books):
    for b, (c, t, _) in books.items():
        K = 1 << b
        np.testing.assert_array_equal(c[::-1], -c)
        assert np.all(np.diff(c) > 0)
        assert t[K // 2 - 1] == 0.0
        np.testing.assert_allclose(t, 0.5 * (c[:-1] + c[1:]), atol=0)


def test_unique_fixed_point(books):
    # f_d is log-concave, so Lloyd's fixed point is unique: any start gives it.
    g = np.random.default_rng(3)
    for b in (2, 3, 4):
        K = 1 << b
        starts = [np.linspace(-0.3, 0.3, K), np.sort(g.uniform(-0.2, 0.2, K))]
        for s in starts:
            c, _, _ = lloyd_max(D, b, init=s)
            np.testing.assert_allclose(c, books[b][0], atol=1e-12)


def test_sphere_monte_carlo(books):
    # Brute force on the sphere: coordinates of uniform unit vectors in R^128.
    # One step of empirical 1-D k-means from the oracle's codebook must leave it
    # in place to Monte-Carlo error, and the empirical distortion must match D.
    g = np.random.default_rng(11)
    x = g.standard_normal((40000, D))
    u = (x / np.linalg.norm(x, axis=1, keepdims=True)).ravel()
    n = u.size
    for b in range(1, 5):
        c, t, Dm = books[b]
        idx = nearest_centroid(u, c)
        err2 = (u - c[idx]) ** 2
        emp = D * err2.mean()
        se = D * err2.std() / math.sqrt(n)
        assert abs(emp - Dm) < 5 * se, (b, emp, Dm, se)
        for i in range(1 << b):
            sel = u[idx == i]
            mc = sel.mean()
            se_i = sel.std() / math.sqrt(sel.size)
            assert abs(mc - c[i]) < 5 * se_i + 1e-12, (b, i, mc, c[i], se_i)

"""Pins of the randomized Walsh-Hadamard rotation (the WHT that
"内存厂商的噩梦来了…" (wuyi.wiki) section 4.3 names as the efficient
replacement of the dense rotation): the oracle's FWHT against the Sylvester
definition, the generated rotation against the oracle's FWHT, and the
distortion it gives against closed forms. CPU only."""
import math

import numpy as np
import pytest

import synth
from oracle import (dequant_mse, dequant_prod, encode_mse, encode_prod, fwht, hadamard_rotate,
                    lloyd_max, nearest_centroid)

D = 128


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128])
def test_fwht_is_the_sylvester_matrix(d):
    H = fwht(np.eye(d))                                   # row i = H e_i (H is symmetric)
    i, j = np.indices((d, d))
    popc = np.vectorize(lambda v: bin(v).count("1"))(i & j)
    np.testing.assert_array_equal(H, (-1.0) ** popc)     # H[i][j] = (-1)^popcount(i & j)
    np.testing.assert_array_equal(H @ H.T, d * np.eye(d))
    # recursive definition H_2n = [[H, H], [H, -H]]
    if d >= 2:
        h = fwht(np.eye(d // 2))
        np.testing.assert_array_equal(H, np.block([[h, h], [h, -h]]))


def test_fwht_linearity_and_involution():
    g = np.random.default_rng(5)
    v, w = g.standard_normal((2, 7, D))
    np.testing.assert_allclose(fwht(2.0 * v - w), 2.0 * fwht(v) - fwht(w), atol=1e-12)
    np.testing.assert_allclose(fwht(fwht(v)), D * v, atol=1e-11)   # H·H = d·I
    with pytest.raises(ValueError):
        fwht(np.ones(12))


@pytest.mark.parametrize("seed", [synth.SEED_HAD_K, synth.SEED_HAD_V, 7])
def test_generated_rotation_is_the_randomized_hadamard_rotation(seed):
    R = synth.hadamard_rotation(D, seed).astype(np.float64)
    s = np.sign(R[0])                                     # the first row of H is all ones
    assert set(np.unique(s)) <= {-1.0, 1.0}
    np.testing.assert_allclose(np.abs(R), 1 / math.sqrt(D), rtol=1e-7)
    U = np.random.default_rng(seed).standard_normal((50, D))
    np.testing.assert_allclose(U @ R.T, hadamard_rotate(U, s), atol=1e-6)
    assert np.abs(R.T @ R - np.eye(D)).max() < 1e-6      # float32-stored factor
    # the signs are balanced draws
    assert abs(s.sum()) < 4 * math.sqrt(D)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_gaussian_distortion_equals_the_haar_value(bits):
    # An isotropic Gaussian x is invariant under every orthogonal map, so
    # H·diag(s)·x/‖x‖ has the same law as a Haar rotation of it: the mean
    # distortion is the Lloyd-Max value D(b) of the exact coordinate law.
    c, t, Dm = lloyd_max(D, bits)
    R = synth.hadamard_rotation(D, 123)
    X = np.random.default_rng(200 + bits).standard_normal((20000, D)) * 0.5
    enc = encode_mse(X, R, c, bits)
    Xt = dequant_mse(enc["codes"], enc["norms"], R, c, bits)
    u = X / np.linalg.norm(X, axis=1, keepdims=True)
    e = ((u - Xt / enc["norms"][:, None]) ** 2).sum(1)
    assert abs(e.mean() - Dm) < 4 * e.std() / math.sqrt(e.size), (bits, e.mean(), Dm)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_basis_vector_closed_form(bits):
    # x = e_k: every rotated coordinate is ±1/√d, so each one takes the
    # centroid c* nearest 1/√d (with its sign) and the distortion is exactly
    # d·(1/√d - c*)², with no averaging over the rotation: a fixed Hadamard
    # rotation maps every basis vector to a flat vector.
    c, t, Dm = lloyd_max(D, bits)
    R = synth.hadamard_rotation(D, 321)
    a = 1 / math.sqrt(D)
    cstar = c[np.argmin(np.abs(c - a))]
    want = D * (a - cstar) ** 2
    for k in (0, 5, 127):
        x = np.zeros((1, D))
        x[0, k] = 3.0
        enc = encode_mse(x, R, c, bits)
        np.testing.assert_array_equal(np.abs(c[enc["idx"][0]]), abs(cstar))
        xt = dequant_mse(enc["codes"], enc["norms"], R, c, bits)[0] / 3.0
        # float32 rotation entries: |y_j| = 1/√d to ~1e-8
        assert abs(((x[0] / 3.0 - xt) ** 2).sum() - want) < 1e-6


@pytest.mark.parametrize("bits", [2, 3])
def test_prod_unbiased_with_hadamard_rotation(bits):
    # The QJL correction is unbiased for any fixed orthogonal Π; with the
    # Hadamard rotation the mean estimate over projection draws matches ⟨y, x⟩.
    c_m = lloyd_max(D, bits - 1)[0]
    R = synth.hadamard_rotation(D, 55).astype(np.float64)
    g = np.random.default_rng(300 + bits)
    x = g.standard_normal(D)
    y = x + g.standard_normal(D)
    nseed = 3000
    est = np.empty(nseed)
    for s in range(nseed):
        S = synth.projection(D, 70_000 + s)
        enc = encode_prod(x[None], R, S, c_m, bits)
        est[s] = dequant_prod(enc["codes"], enc["norms"], enc["qjl"], enc["gammas"], R, S, c_m, bits)[0] @ y
    se = est.std() / math.sqrt(nseed)
    assert abs(est.mean() - x @ y) < 4 * se, (est.mean(), x @ y, se)
    # and the mse part alone is the same nearest-centroid code as the FWHT form
    u = x / np.linalg.norm(x)
    np.testing.assert_array_equal(nearest_centroid(R @ u, c_m),
                                  nearest_centroid(hadamard_rotate(u, np.sign(R[0])), c_m))

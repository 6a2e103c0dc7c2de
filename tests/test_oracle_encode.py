"""Pins of the oracle's encode / dequant / packing against worked examples,
brute force, invariants of the random rotation and the statistical claims the
pages make (distortion, mse bias, prod unbiasedness and variance). CPU only."""
import math
import os

import numpy as np
import pytest
from scipy import stats

import synth
from oracle import (coord_mass, decode_attention, dequant_mse, dequant_prod, encode_mse,
                    encode_prod, lloyd_max, nearest_centroid, pack_codes, pack_signs,
                    unpack_codes, unpack_signs)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
D = 128


def _kv(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, *v = line.split()
                out[k] = v
    return out


@pytest.fixture(scope="module")
def books():
    return {b: lloyd_max(D, b) for b in range(0, 5)}


def test_pack_worked_example():
    g = _kv("pack_b3_worked_example.txt")
    bits = int(g["bits"][0])
    codes = np.array([[int(c) for c in g["codes"]]])
    want = bytes(int(b, 16) for b in g["bytes"])
    got = pack_codes(codes, bits)
    assert got.tobytes() == want
    np.testing.assert_array_equal(unpack_codes(got, codes.shape[1], bits), codes)


def test_pack_signs_example():
    g = _kv("pack_signs_example.txt")
    z = np.array([[float(v) for v in g["z"]]])
    want = bytes(int(b, 16) for b in g["bytes"])
    got = pack_signs(z)
    assert got.tobytes() == want
    np.testing.assert_array_equal(unpack_signs(got, z.shape[1]), np.where(z >= 0, 1.0, -1.0))


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_pack_roundtrip_and_bit_positions(bits):
    g = np.random.default_rng(bits)
    idx = g.integers(0, 1 << bits, size=(50, D))
    p = pack_codes(idx, bits)
    assert p.shape == (50, D * bits // 8)
    np.testing.assert_array_equal(unpack_codes(p, D, bits), idx)
    # Every 32 codes fill exactly `bits` 32-bit words: check one code by
    # reading its bits out of the little-endian word stream by hand.
    words = p.view("<u4")
    for v, j in [(0, 0), (3, 31), (7, 77), (49, 127)]:
        pos = j * bits
        val = 0
        for k in range(bits):
            w, o = divmod(pos + k, 32)
            val |= ((int(words[v, w]) >> o) & 1) << k
        assert val == idx[v, j]


@pytest.mark.parametrize("d", [4, 8, 16, 128])
def test_nearest_centroid_brute_force_and_boundaries(d):
    g = np.random.default_rng(d)
    for b in (1, 2, 3, 4):
        c, t, _ = lloyd_max(d, b)
        y = g.standard_normal((1000, d)) / math.sqrt(d)
        idx = nearest_centroid(y, c)
        # brute force over every centroid with explicit loops
        bf = np.zeros_like(idx)
        for (i, j), v in np.ndenumerate(y):
            best, bi = np.inf, -1
            for k, ck in enumerate(c):
                e = abs(v - ck)
                if e < best:
                    best, bi = e, k
            bf[i, j] = bi
        np.testing.assert_array_equal(idx, bf)
        # boundary search: #{i : t_i < y}
        np.testing.assert_array_equal(idx, np.sum(y[..., None] > t, axis=-1))


def test_joint_brute_force_tiny():
    # d = 4, 2 bits: search all 4^4 code vectors for the reconstruction closest
    # to Π u; it must be the per-coordinate nearest-centroid encoding.
    d, b = 4, 2
    c, _, _ = lloyd_max(d, b)
    rot = synth.rotation(d, 5)
    X = np.random.default_rng(1).standard_normal((200, d))
    enc = encode_mse(X, rot, c, b)
    grid = np.array(np.meshgrid(*[np.arange(4)] * d, indexing="ij")).reshape(d, -1).T
    recon = c[grid] @ rot.astype(np.float64)            # Πᵀ c[idx], every code vector
    u = X / np.linalg.norm(X, axis=1, keepdims=True)
    best = np.argmin(((u[:, None, :] - recon[None]) ** 2).sum(-1), axis=1)
    np.testing.assert_array_equal(grid[best], enc["idx"])


def test_rotation_is_orthogonal():
    R = synth.rotation(D, synth.SEED_ROT_K).astype(np.float64)
    assert np.abs(R.T @ R - np.eye(D)).max() < 1e-6      # float32-stored factor
    g = np.random.default_rng(0).standard_normal((D, D))
    q, r = np.linalg.qr(g)
    q = q * np.sign(np.diag(r))
    assert np.abs(q.T @ q - np.eye(D)).max() < 1e-12


def test_rotated_coordinate_law_ks():
    # For a fixed unit u, (Π u)_0 over independent rotation seeds follows f_d
    # ("Trick đầu tiên…": a randomly rotated unit vector has coordinates with
    # density C(1-x²)^((d-3)/2)). KS test against the CDF of that law.
    d = 64
    u = np.zeros(d)
    u[3] = 1.0
    vals = np.array([(synth.rotation(d, 10_000 + s).astype(np.float64) @ u)[0] for s in range(1500)])
    cdf = lambda x: coord_mass(-1.0, x, d)
    assert stats.kstest(vals, cdf).pvalue > 1e-3


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_mse_distortion_monte_carlo(books, bits):
    c, t, Dm = books[bits]
    rot = synth.rotation(D, 77)
    X = np.random.default_rng(bits).standard_normal((20000, D)) * 3.0
    enc = encode_mse(X, rot, c, bits)
    Xt = dequant_mse(enc["codes"], enc["norms"], rot, c, bits)
    u = X / np.linalg.norm(X, axis=1, keepdims=True)
    ut = Xt / enc["norms"][:, None]
    e = ((u - ut) ** 2).sum(1)
    assert abs(e.mean() - Dm) < 4 * e.std() / math.sqrt(e.size)
    assert 1 / 4 ** bits <= e.mean() <= (math.sqrt(3) * math.pi / 2) / 4 ** bits


def test_mse_inner_product_bias(books):
    # E_Π ⟨y, x̃⟩ = (1 - D(b)) ⟨y, x⟩: the mse quantizer shrinks inner products
    # ("Vấn đề của inner product: bias không phải MSE"); at b = 1 the factor is
    # ≈ 2/π ("内存厂商的噩梦来了…" section 4.2). The factor is exact for a
    # Lloyd-Max codebook: E⟨u,ũ⟩ = E‖ũ‖² = 1 - D by the centroid condition.
    d = 32
    g = np.random.default_rng(5)
    x = g.standard_normal(d)
    y = x + 0.5 * g.standard_normal(d)
    rots = [synth.rotation(d, 20_000 + s) for s in range(3000)]
    for b in (1, 2, 3):
        c, _, Dm = lloyd_max(d, b)
        est = np.empty(len(rots))
        for s, R in enumerate(rots):
            enc = encode_mse(x[None], R, c, b)
            est[s] = dequant_mse(enc["codes"], enc["norms"], R, c, b)[0] @ y
        ratio = est / (x @ y)
        assert abs(ratio.mean() - (1 - Dm)) < 4 * ratio.std() / math.sqrt(ratio.size), (b, ratio.mean(), 1 - Dm)
    c1, _, D1 = lloyd_max(D, 1)
    assert abs((1 - D1) - 2 / math.pi) < 3e-3


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_prod_unbiased_and_variance(books, bits):
    # QJL on the residual makes ⟨y, x̃⟩ unbiased over the projection draw
    # ("TurboQuant của Google…", QJL section: E⟨y, x̃⟩ = ⟨y, x⟩), with variance
    # [(π/2)γ²‖y‖² - ⟨y,r⟩²]/d·n², ≤ (π/(2d))‖y‖² at γ = 1.
    c_m = books[bits - 1][0]
    rot = synth.rotation(D, 99).astype(np.float64)
    g = np.random.default_rng(100 + bits)
    x = g.standard_normal(D) * 2.0
    y = x + g.standard_normal(D)
    n = np.linalg.norm(x)
    u = x / n
    idx = nearest_centroid(rot @ u, c_m)
    r = u - c_m[idx] @ rot
    gam = np.linalg.norm(r)
    nseed = 6000
    est = np.empty(nseed)
    for s in range(nseed):
        S = synth.projection(D, 50_000 + s)
        enc = encode_prod(x[None], rot, S, c_m, bits)
        xt = dequant_prod(enc["codes"], enc["norms"], enc["qjl"], enc["gammas"], rot, S, c_m, bits)[0]
        est[s] = xt @ y
    truth = x @ y
    se = est.std() / math.sqrt(nseed)
    assert abs(est.mean() - truth) < 4 * se, (bits, est.mean(), truth, se)
    var_pred = ((math.pi / 2) * gam ** 2 * (y @ y) - (y @ r) ** 2) / D * n ** 2
    assert abs(est.var() / var_pred - 1) < 4 * math.sqrt(2 / nseed) + 0.02
    if bits == 1:
        assert abs(gam - 1) < 1e-12
        assert var_pred <= math.pi / (2 * D) * (y @ y) * n ** 2


def test_mse_biased_prod_not_at_one_bit(books):
    # Figure 1 of the paper as described on omelet.tech: at b = 1 the mse
    # inner-product error is shifted, prod's is centred at 0. Over random unit
    # x and correlated y with fixed Π, S.
    rot = synth.rotation(D, 3)
    S = synth.projection(D, 4)
    g = np.random.default_rng(8)
    X = g.standard_normal((4000, D))
    Y = X + g.standard_normal((4000, D))
    c1 = books[1][0]
    e1 = encode_mse(X, rot, c1, 1)
    m = (dequant_mse(e1["codes"], e1["norms"], rot, c1, 1) * Y).sum(1) - (X * Y).sum(1)
    c0 = books[0][0]
    e2 = encode_prod(X, rot, S, c0, 1)
    p = (dequant_prod(e2["codes"], e2["norms"], e2["qjl"], e2["gammas"], rot, S, c0, 1) * Y).sum(1) - (X * Y).sum(1)
    assert m.mean() < -10 * m.std() / math.sqrt(m.size)
    assert abs(p.mean()) < 4 * p.std() / math.sqrt(p.size)


def test_tie_at_zero_goes_to_lower_index(books):
    # y = 0 sits exactly on the middle boundary: both middle centroids are at
    # the same distance and the lower index wins.
    for b in (1, 2, 3, 4):
        c = books[b][0]
        assert nearest_centroid(np.zeros(3), c).tolist() == [(1 << b) // 2 - 1] * 3


def test_zero_vector(books):
    c, _, _ = books[3]
    rot = synth.rotation(D, 1)
    S = synth.projection(D, 2)
    X = np.zeros((2, D))
    X[1, 5] = 1.0
    enc = encode_mse(X, rot, c, 3)
    assert enc["norms"][0] == 0.0
    assert np.all(enc["idx"][0] == 3)          # y = 0 → lower of the two middle centroids
    assert np.all(dequant_mse(enc["codes"], enc["norms"], rot, c, 3)[0] == 0.0)
    cm = books[2][0]
    e2 = encode_prod(X, rot, S, cm, 3)
    assert np.all(dequant_prod(e2["codes"], e2["norms"], e2["qjl"], e2["gammas"], rot, S, cm, 3)[0] == 0.0)

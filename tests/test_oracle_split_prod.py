"""Pins of the oracle's outlier-channel split with prod keys ("TurboQuant của
Google…" (omelet.tech) section "Thực nghiệm: 3.5 bit…" for the two groups at
one bit apart; its QJL section for the prod quantizer): the bit budget
against the printed labels, unbiasedness of inner products over the two
sketch draws, the variance's closed form with each group's own dimension in
the correction scale, the sketch bits' positions, and the zero vector.
CPU only."""
import math

import numpy as np
import pytest

import synth
from oracle import (dequant_split_prod, encode_split_prod, lloyd_max, nearest_centroid, pack_split,
                    split_positions, unpack_signs)

D = 128


def _books(bits):
    return lloyd_max(32, bits)[0], lloyd_max(96, bits - 1)[0]


@pytest.mark.parametrize("bits,label", [(2, 2.5), (3, 3.5)])
def test_bit_budget_matches_the_printed_labels(bits, label):
    # outlier group prod at bits + 1 (bits of codes + 1 sketch bit), regular
    # at bits (bits - 1 + 1): 32·(bits + 1) + 96·bits bits per vector, the
    # printed average once two 16-bit norms are added, as for the mse split
    codes = pack_split(np.zeros((1, D), np.int64), bits - 1).shape[1]
    total = 8 * codes + D
    assert total == 32 * (bits + 1) + 96 * bits
    assert (total + 2 * 16) / D == label


def _setup(seed, bits):
    c = synth.split_constants(D)
    g = np.random.default_rng(seed)
    x = g.standard_normal(D)
    x[c["ch_k"][:4]] *= 8.0
    y = x + g.standard_normal(D)
    return c, x, y


@pytest.mark.parametrize("bits", [2, 3])
def test_inner_products_unbiased_with_the_groupwise_variance(bits):
    # Over independent Gaussian S_o (32×32) and S_r (96×96), E⟨y, x̃⟩ = ⟨y, x⟩
    # (each group's estimate is unbiased), and the variance is the sum of the
    # groups' [(π/2) γ_g² ‖y_g‖² - ⟨y_g, r_g⟩²] n_g² / d_g with d_o = 32 and
    # d_r = 96: a wrong dimension in either correction scale, a wrong sign or
    # a sketch read at the other group's positions breaks one of the two.
    c, x, y = _setup(7 + bits, bits)
    ch = np.asarray(c["ch_k"])
    ch_r = np.setdiff1d(np.arange(D), ch)
    co, cr = _books(bits)
    ro, rr = c["rk_o"].astype(np.float64), c["rk_r"].astype(np.float64)
    var = 0.0
    for chs, R, cb, dg in ((ch, ro, co, 32), (ch_r, rr, cr, 96)):
        xg, yg = x[chs], y[chs]
        n = np.linalg.norm(xg)
        u = xg / n
        r = u - cb[nearest_centroid(R @ u, cb)] @ R
        gam = np.linalg.norm(r)
        var += ((math.pi / 2) * gam ** 2 * (yg @ yg) - (yg @ r) ** 2) / dg * n ** 2
    nseed = 4000
    est = np.empty(nseed)
    for s in range(nseed):
        So = synth.projection(32, 90_000 + s)
        Sr = synth.projection(96, 190_000 + s)
        e = encode_split_prod(x[None], ch, ro, rr, So, Sr, co, cr, bits)
        xt = dequant_split_prod(e["codes"], e["norms"], e["qjl"], e["gammas"], ch, ro, rr, So, Sr, co, cr, bits)[0]
        est[s] = xt @ y
    se = est.std() / math.sqrt(nseed)
    assert abs(est.mean() - x @ y) < 4 * se, (est.mean(), x @ y, se)
    assert abs(est.var() / var - 1) < 4 * math.sqrt(2 / nseed) + 0.02, (est.var(), var)


def test_sketch_bits_sit_at_the_group_positions():
    # the outlier group's sketch values go to positions p mod 8 < 2 in group
    # order, the regular group's to the others: flipping the sign of S_o
    # flips exactly the outlier positions' bits
    bits = 3
    c, x, _ = _setup(21, bits)
    ch = np.asarray(c["ch_k"])
    co, cr = _books(bits)
    ro, rr = c["rk_o"], c["rk_r"]
    So, Sr = synth.projection(32, 5), synth.projection(96, 6)
    a = unpack_signs(encode_split_prod(x[None], ch, ro, rr, So, Sr, co, cr, bits)["qjl"], D)[0]
    b = unpack_signs(encode_split_prod(x[None], ch, ro, rr, -So, Sr, co, cr, bits)["qjl"], D)[0]
    P_o, P_r = split_positions(D)
    flipped = np.nonzero(a != b)[0]
    assert set(flipped.tolist()) == set(P_o.tolist())
    e = encode_split_prod(x[None], ch, ro, rr, So, Sr, co, cr, bits)
    assert np.array_equal(a[P_o], np.where(e["z_o"][0] >= 0, 1, -1))
    assert np.array_equal(a[P_r], np.where(e["z_r"][0] >= 0, 1, -1))


def test_zero_vector_and_empty_group():
    # a zero vector decodes to zero; a vector with no energy in the regular
    # channels decodes to zero there (n_r = 0) and keeps the outlier part
    bits = 2
    c, x, _ = _setup(31, bits)
    ch = np.asarray(c["ch_k"])
    ch_r = np.setdiff1d(np.arange(D), ch)
    co, cr = _books(bits)
    ro, rr = c["rk_o"], c["rk_r"]
    So, Sr = synth.projection(32, 7), synth.projection(96, 8)
    X = np.stack([np.zeros(D), x.copy()])
    X[1, ch_r] = 0.0
    e = encode_split_prod(X, ch, ro, rr, So, Sr, co, cr, bits)
    xt = dequant_split_prod(e["codes"], e["norms"], e["qjl"], e["gammas"], ch, ro, rr, So, Sr, co, cr, bits)
    assert np.all(xt[0] == 0)
    assert np.all(xt[1, ch_r] == 0) and e["norms"][1, 1] == 0
    assert np.linalg.norm(xt[1, ch] - X[1, ch]) < 0.5 * np.linalg.norm(X[1, ch])

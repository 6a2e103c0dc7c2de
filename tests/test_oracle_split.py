"""Pins of the oracle's outlier-channel split ("TurboQuant của Google…"
(omelet.tech) section "Thực nghiệm: 3.5 bit…": 32 outlier channels at one bit
more than the other 96, two independent TurboQuant instances): the code
string's size against the printed counts, a hand-derived worked example of
its layout, reduction to the plain quantizer on each group, and each group's
distortion against the Lloyd-Max value for its dimension. CPU only."""
import math
import os

import numpy as np
import pytest

import synth
from oracle import (codebook_mse, dequant_mse, dequant_split, encode_mse, encode_split, lloyd_max, pack_split,
                    split_positions, unpack_split)

D = 128
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _books(bits):
    co, to, _ = lloyd_max(32, bits + 1)
    cr, tr, _ = lloyd_max(96, bits)
    return co, to, cr, tr


@pytest.mark.parametrize("bits,label", [(2, 2.5), (3, 3.5)])
def test_code_string_size_matches_the_printed_counts(bits, label):
    # 32 channels at bits + 1 and 96 at bits, as printed: for "2.5-bit"
    # 32·3 + 96·2 = 288 code bits; with two 16-bit group norms the average
    # per channel is the printed label.
    n = pack_split(np.zeros((1, D), np.int64), bits).shape[1]
    assert 8 * n == 32 * (bits + 1) + 96 * bits
    assert (8 * n + 2 * 16) / D == label
    P_o, P_r = split_positions(D)
    assert len(P_o) == 32 and len(P_r) == 96 and set(P_o) | set(P_r) == set(range(D))


def test_worked_example_b2():
    spec = {}
    for line in open(os.path.join(GOLDEN, "pack_split_b2.txt")):
        if line.strip() and not line.startswith("#"):
            k, v = line.split(maxsplit=1)
            spec[k] = v.split()
    bits = int(spec["bits"][0])
    P_o, P_r = split_positions(D)
    idx = np.zeros((1, D), np.int64)
    idx[0, P_o] = int(spec["outlier_code"][0])
    idx[0, P_r] = int(spec["regular_code"][0])
    want = np.array([int(b, 16) for b in spec["bytes"]], np.uint8)
    np.testing.assert_array_equal(pack_split(idx, bits)[0], want)
    np.testing.assert_array_equal(unpack_split(want[None], bits), idx)


def test_single_codes_land_where_the_layout_says():
    # b = 2: outlier coordinate 5 sits at position 17 (chunk 2, slot 1); chunk
    # 2 starts at stream bit 36, slot 1 at +3, so code 7 sets bits 39-41:
    # bit 7 of byte 4 and bits 0-1 of byte 5.
    P_o, P_r = split_positions(D)
    assert P_o[5] == 17
    idx = np.zeros((1, D), np.int64)
    idx[0, 17] = 7
    b = pack_split(idx, 2)[0]
    assert b[4] == 0x80 and b[5] == 0x03 and np.count_nonzero(b) == 2
    # b = 3: position 0 (4 bits) code 15 fills byte 0; position 2 (the first
    # regular one, 3 bits at stream bit 8) code 5 gives byte 1 = 0b101.
    idx = np.zeros((1, D), np.int64)
    idx[0, 0] = 15
    idx[0, 2] = 5
    b = pack_split(idx, 3)[0]
    assert b[0] == 0x0F and b[1] == 0x05 and np.count_nonzero(b) == 2
    # round trip of random codes at both widths
    g = np.random.default_rng(3)
    for bits in (2, 3):
        idx = np.zeros((50, D), np.int64)
        idx[:, P_o] = g.integers(0, 2 ** (bits + 1), (50, 32))
        idx[:, P_r] = g.integers(0, 2 ** bits, (50, 96))
        np.testing.assert_array_equal(unpack_split(pack_split(idx, bits), bits), idx)


@pytest.mark.parametrize("bits", [2, 3])
def test_each_group_is_the_plain_quantizer(bits):
    c = synth.split_constants(D)
    co, _, cr, _ = _books(bits)
    ch_o = c["ch_k"]
    ch_r = np.setdiff1d(np.arange(D), ch_o)
    g = np.random.default_rng(10 + bits)
    X = g.standard_normal((300, D))
    enc = encode_split(X, ch_o, c["rk_o"], c["rk_r"], co, cr, bits)
    P_o, P_r = split_positions(D)
    # the plain quantizer on each group's raw channels gives its codes and norm
    eo = encode_mse(X[:, ch_o], c["rk_o"], co, bits + 1)
    er = encode_mse(X[:, ch_r], c["rk_r"], cr, bits)
    np.testing.assert_array_equal(enc["idx"][:, P_o], eo["idx"])
    np.testing.assert_array_equal(enc["idx"][:, P_r], er["idx"])
    np.testing.assert_allclose(enc["norms"][:, 0], np.linalg.norm(X[:, ch_o], axis=1), rtol=1e-13)
    np.testing.assert_allclose(enc["norms"][:, 1], np.linalg.norm(X[:, ch_r], axis=1), rtol=1e-13)
    Xt = dequant_split(enc["codes"], enc["norms"], ch_o, c["rk_o"], c["rk_r"], co, cr, bits)
    np.testing.assert_allclose(Xt[:, ch_o], dequant_mse(eo["codes"], eo["norms"], c["rk_o"], co, bits + 1),
                               atol=1e-12)
    np.testing.assert_allclose(Xt[:, ch_r], dequant_mse(er["codes"], er["norms"], c["rk_r"], cr, bits), atol=1e-12)
    # a vector whose regular channels are zero reconstructs to zero there
    Z = X.copy()
    Z[:, ch_r] = 0.0
    ez = encode_split(Z, ch_o, c["rk_o"], c["rk_r"], co, cr, bits)
    assert np.all(ez["norms"][:, 1] == 0)
    Zt = dequant_split(ez["codes"], ez["norms"], ch_o, c["rk_o"], c["rk_r"], co, cr, bits)
    assert np.all(Zt[:, ch_r] == 0)


@pytest.mark.parametrize("bits", [2, 3])
def test_group_distortion_is_the_lloyd_max_value(bits):
    # Each group is a TurboQuant-mse instance in its own dimension: on
    # Gaussian data its unit vector's mean squared error is D(d_g, b_g).
    c = synth.split_constants(D)
    co, to, cr, tr = _books(bits)
    ch_o = c["ch_k"]
    ch_r = np.setdiff1d(np.arange(D), ch_o)
    X = np.random.default_rng(20 + bits).standard_normal((20000, D))
    enc = encode_split(X, ch_o, c["rk_o"], c["rk_r"], co, cr, bits)
    Xt = dequant_split(enc["codes"], enc["norms"], ch_o, c["rk_o"], c["rk_r"], co, cr, bits)
    for ch, j, cb, tb, dg, bg in ((ch_o, 0, co, to, 32, bits + 1), (ch_r, 1, cr, tr, 96, bits)):
        n = enc["norms"][:, j:j + 1]
        e = np.sum((X[:, ch] / n - Xt[:, ch] / n) ** 2, axis=1)
        want = codebook_mse(cb, tb, dg)
        assert abs(e.mean() - want) < 4 * e.std() / math.sqrt(e.size), (dg, bg, e.mean(), want)


def test_split_helps_on_outlier_channels():
    # On data whose listed channels are 4x larger, 3 bits on those channels
    # and 2 on the rest reconstructs better than 2 bits everywhere.
    c = synth.split_constants(D)
    X = synth.split_kv(1, 1, 4000, D, 31, c["ch_k"], dtype="fp32")[0, 0].astype(np.float64)
    co, _, cr, _ = _books(2)
    enc = encode_split(X, c["ch_k"], c["rk_o"], c["rk_r"], co, cr, 2)
    e_split = np.sum((X - dequant_split(enc["codes"], enc["norms"], c["ch_k"], c["rk_o"], c["rk_r"], co, cr, 2)) ** 2)
    R = synth.rotation(D, 55)
    c2, _, _ = lloyd_max(D, 2)
    eu = encode_mse(X, R, c2, 2)
    e_uni = np.sum((X - dequant_mse(eu["codes"], eu["norms"], R, c2, 2)) ** 2)
    assert e_split < 0.8 * e_uni, (e_split, e_uni)

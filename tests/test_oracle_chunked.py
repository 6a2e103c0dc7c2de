"""Pins of the oracle's reading of vectors longer than 128 coordinates
("内存厂商的噩梦来了…" (wuyi.wiki) section 6.4: search over d = 200 GloVe
vectors, index build for d = 1536): zero padding to a multiple of 128, chunks
of 128 quantized on their own, the estimate summed over chunks. Checked
against a worked layout, the exact identities of zero padding, the
codebook's closed-form distortion (which a wrong cut or a transposed chunk
would break) and the unbiasedness of the summed prod estimate. CPU only."""
import math

import numpy as np
import pytest

import synth
from oracle import (chunk_vectors, dequant_mse, dequant_prod, encode_mse, encode_prod, lloyd_max, search_topk,
                    unchunk_vectors)

W = 128


def test_chunk_layout_worked_example():
    # row i holds 1000·i + j at coordinate j: chunk c of row i must hold
    # 1000·i + 128c .. 1000·i + 128c + 127, zeros past the vector's length
    n, D = 3, 200
    X = 1000.0 * np.arange(n)[:, None] + np.arange(D)[None, :]
    Xc = chunk_vectors(X, W)
    assert Xc.shape == (2, n, W)
    for i in range(n):
        assert Xc[0, i].tolist() == [1000.0 * i + j for j in range(128)]
        assert Xc[1, i, :72].tolist() == [1000.0 * i + j for j in range(128, 200)]
        assert np.all(Xc[1, i, 72:] == 0)
    assert unchunk_vectors(Xc).shape == (n, 256)
    np.testing.assert_array_equal(unchunk_vectors(Xc)[:, :D], X)


@pytest.mark.parametrize("D,C", [(1, 1), (127, 1), (128, 1), (129, 2), (200, 2), (256, 2), (1536, 12)])
def test_chunk_counts_and_identities(D, C):
    g = np.random.default_rng(D)
    X = g.standard_normal((5, D))
    Q = g.standard_normal((4, D))
    Xc, Qc = chunk_vectors(X, W), chunk_vectors(Q, W)
    assert Xc.shape == (C, 5, W)
    # zero padding keeps norms and inner products: Σ_c ‖x_c‖² = ‖x‖²,
    # Σ_c ⟨q_c, x_c⟩ = ⟨q, x⟩
    np.testing.assert_allclose((Xc ** 2).sum(axis=(0, 2)), (X ** 2).sum(1), rtol=1e-13)
    np.testing.assert_allclose(np.einsum("cqw,cxw->qx", Qc, Xc), Q @ X.T, rtol=1e-12, atol=1e-12)
    # D = 128: one chunk, the vectors themselves
    if D == W:
        np.testing.assert_array_equal(Xc[0], X)


@pytest.mark.parametrize("D,bits", [(200, 2), (200, 4), (1536, 3)])
def test_chunked_mse_distortion_is_the_codebooks(D, bits):
    # Each chunk is a vector of R^128 of its own, rotated uniformly onto the
    # sphere, so its relative error has the codebook's expectation D(b); the
    # whole vector's error ‖x - x̃‖² / ‖x‖² is the chunk errors weighted by
    # ‖x_c‖² / ‖x‖², with the same expectation D(b).
    c, _, Dm = lloyd_max(W, bits)
    rot = synth.rotation(W, 300 + bits)
    n = 6000 if D == 200 else 800
    X = np.random.default_rng(D + bits).standard_normal((n, D))
    Xc = chunk_vectors(X, W)
    parts = []
    for ch in Xc:
        enc = encode_mse(ch, rot, c, bits)
        parts.append(dequant_mse(enc["codes"], enc["norms"], rot, c, bits))
    Xt = unchunk_vectors(np.stack(parts))
    e = ((unchunk_vectors(Xc) - Xt) ** 2).sum(1) / (X ** 2).sum(1)
    assert abs(e.mean() - Dm) < 4 * e.std() / math.sqrt(e.size), (e.mean(), Dm)


def test_chunked_prod_sum_is_unbiased():
    # the summed prod estimate Σ_c ⟨q_c, x̃_c⟩ is unbiased over the
    # projection draw (each chunk's is, and the sum is linear)
    D, bits = 200, 2
    c_m = lloyd_max(W, bits - 1)[0]
    rot = synth.rotation(W, 31)
    g = np.random.default_rng(32)
    x = g.standard_normal(D)
    y = x + g.standard_normal(D)
    xc, yc = chunk_vectors(x[None], W), chunk_vectors(y[None], W)
    nseed = 3000
    est = np.empty(nseed)
    for s in range(nseed):
        S = synth.projection(W, 70_000 + s)
        tot = 0.0
        for cx, cy in zip(xc, yc):
            enc = encode_prod(cx, rot, S, c_m, bits)
            tot += dequant_prod(enc["codes"], enc["norms"], enc["qjl"], enc["gammas"], rot, S, c_m, bits)[0] @ cy[0]
        est[s] = tot
    se = est.std() / math.sqrt(nseed)
    assert abs(est.mean() - x @ y) < 4 * se, (est.mean(), x @ y, se)


def test_chunked_search_finds_the_true_top1_at_d200():
    # recall 1@10 of the chunked prod-4 search on Gaussian d = 200 data is
    # high, and it is 1 at k = n
    D, bits, n, nq = 200, 4, 3000, 40
    g = np.random.default_rng(41)
    X = g.standard_normal((n, D))
    Q = g.standard_normal((nq, D))
    true1 = np.argmax(Q @ X.T, axis=1)
    c_m = lloyd_max(W, bits - 1)[0]
    rot, S = synth.rotation(W, 42), synth.projection(W, 43)
    parts = []
    for ch in chunk_vectors(X, W):
        enc = encode_prod(ch, rot, S, c_m, bits)
        parts.append(dequant_prod(enc["codes"], enc["norms"], enc["qjl"], enc["gammas"], rot, S, c_m, bits))
    Xt = unchunk_vectors(np.stack(parts))
    Qp = unchunk_vectors(chunk_vectors(Q, W))
    ix10 = search_topk(Qp, Xt, 10)[1]
    rec = np.mean([true1[i] in ix10[i] for i in range(nq)])
    assert rec > 0.9, rec
    ixn = search_topk(Qp, Xt, n)[1]
    assert all(true1[i] in ixn[i] for i in range(nq))

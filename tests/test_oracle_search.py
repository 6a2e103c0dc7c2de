"""Pins of the oracle's inner-product search ("内存厂商的噩梦来了…" (wuyi.wiki)
section 6.4: nearest-neighbour search by inner product over TurboQuant-encoded
vectors, scored by recall 1@k): brute force on tiny inputs, tie order, the
full sort at k = n, and recall against the unquantized search. CPU only."""
import math

import numpy as np
import pytest

import synth
from oracle import dequant_prod, encode_prod, lloyd_max, recall_1_at_k, search_topk

D = 128


def test_search_has_the_defining_properties():
    # Integer-valued data, so exact ties are common. For each query the k
    # results are distinct, their scores do not increase, every row left out
    # scores at most the k-th score, and a left-out row that ties the k-th
    # score has a larger index than every returned row with that score.
    g = np.random.default_rng(1)
    for n, k in ((1, 1), (5, 2), (9, 9), (40, 7), (200, 25)):
        Q = g.integers(-2, 3, (4, 5)).astype(np.float64)
        X = g.integers(-2, 3, (n, 5)).astype(np.float64)
        sc, ix = search_topk(Q, X, k)
        for i in range(Q.shape[0]):
            s = X @ Q[i]
            got = ix[i].tolist()
            assert len(set(got)) == k
            np.testing.assert_array_equal(sc[i], s[got])
            assert all(sc[i][a] >= sc[i][a + 1] for a in range(k - 1))
            kth = sc[i][-1]
            for j in set(range(n)) - set(got):
                assert s[j] <= kth
                if s[j] == kth:
                    assert all(j > r for r in got if s[r] == kth)
            for a in range(k - 1):                  # equal scores: ascending index
                if sc[i][a] == sc[i][a + 1]:
                    assert got[a] < got[a + 1]


def test_ties_go_to_the_lower_index_and_k_equal_n_is_a_full_sort():
    X = np.array([[1.0, 0], [0, 1.0], [1.0, 0], [0.5, 0], [1.0, 0]])
    Q = np.array([[1.0, 0.0]])
    sc, ix = search_topk(Q, X, 5)
    assert ix[0].tolist() == [0, 2, 4, 3, 1]
    np.testing.assert_array_equal(sc[0], [1, 1, 1, 0.5, 0])


def test_recall_definition():
    assert recall_1_at_k([3, 7], [[1, 3], [2, 5]]) == 0.5
    assert recall_1_at_k([3], [[3]]) == 1.0


@pytest.mark.parametrize("bits", [2, 4])
def test_recall_of_the_packed_search_grows_with_k_and_bits(bits):
    # Gaussian database and queries: the search over the dequantized prod
    # vectors finds the true top-1 more often as k grows, always when k = n,
    # and (statistically) more often at 4 bits than at 2.
    g = np.random.default_rng(10 + bits)
    n, nq = 2000, 60
    X = g.standard_normal((n, D))
    Q = g.standard_normal((nq, D))
    true1 = np.argmax(Q @ X.T, axis=1)
    rot = synth.rotation(D, 5)
    S = synth.projection(D, 6)
    c = lloyd_max(D, bits - 1)[0]
    enc = encode_prod(X, rot, S, c, bits)
    Xt = dequant_prod(enc["codes"], enc["norms"], enc["qjl"], enc["gammas"], rot, S, c, bits)
    recs = [recall_1_at_k(true1, search_topk(Q, Xt, k)[1]) for k in (1, 4, 16, 64, n)]
    assert all(a <= b for a, b in zip(recs, recs[1:])), recs
    assert recs[-1] == 1.0
    assert recs[2] > (0.6 if bits == 2 else 0.9), recs
    # unquantized search finds it at k = 1
    assert recall_1_at_k(true1, search_topk(Q, X, 1)[1]) == 1.0

"""GPU parity of tq_encode against the oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import synth
from kv_cache_vector_06_amd import _lib as L
from kv_cache_vector_06_amd import torch_api as T
from gpu_util import (DEV, assert_guards, book, check_encode, gpu_packed_arrays, guarded_packed, oracle_encode, say,
                      to_gpu_x)
from oracle import encode_mse, encode_prod, unpack_codes, unpack_signs

pytestmark = pytest.mark.gpu

CASES = [(b, v, dt) for v in ("mse", "prod") for b in (1, 2, 3, 4) for dt in ("bf16", "fp32")]


@pytest.fixture(scope="module")
def consts():
    return synth.constants(128)


@pytest.mark.parametrize("bits,variant,dtype", CASES)
def test_encode_parity(consts, bits, variant, dtype):
    Rk, _, S = consts
    n = 4096 + 37                                   # several tiles and a ragged tail
    X = synth.outlier_kv(1, 1, n, 128, seed=100 + bits, dtype=dtype)[0, 0]
    say("encode", bits, variant, dtype, n)
    q = T.Quantizer(Rk, bits, variant, S if variant == "prod" else None, DEV)
    p = T.encode(q, to_gpu_x(X, dtype), guarded_packed(q, n))
    assert_guards(p)
    st = check_encode(gpu_packed_arrays(p, q), oracle_encode(X, Rk, S, bits, variant), bits, variant)
    say(st)


@pytest.mark.parametrize("bits,variant,dtype", CASES)
def test_encode_parity_hadamard(bits, variant, dtype):
    # Randomized Walsh-Hadamard rotation: exact ±1 operands, 1/√d in fp32.
    # Outlier-channel data, plus a zero row and one-hot rows (which this
    # rotation maps to flat vectors of ±1/√d).
    Rk, _, S = synth.hadamard_constants(128)
    n = 2048 + 37
    X = synth.outlier_kv(1, 1, n, 128, seed=400 + bits, dtype=dtype)[0, 0].copy()
    X[0] = 0.0
    X[1] = 0.0
    X[1, 5] = 3.0
    X[2] = 0.0
    X[2, 127] = -0.5
    say("encode hadamard", bits, variant, dtype, n)
    q = T.Quantizer(Rk, bits, variant, S if variant == "prod" else None, DEV, "hadamard")
    xg = to_gpu_x(X, dtype)
    p = T.encode(q, xg, guarded_packed(q, n))
    assert_guards(p)
    g = gpu_packed_arrays(p, q)
    st = check_encode(g, oracle_encode(X, Rk, S, bits, variant), bits, variant)
    say(st)
    ps = T.encode(q, xg[:37], guarded_packed(q, 37))          # the row-tile encoder
    assert_guards(ps)
    small = gpu_packed_arrays(ps, q)
    for k in g:
        np.testing.assert_array_equal(small[k], g[k][:37])


@pytest.mark.parametrize("variant", ["mse", "prod"])
def test_encode_edge_cases(consts, variant):
    Rk, _, S = consts
    g = np.random.default_rng(5)
    X = g.standard_normal((70, 128)).astype(np.float32)
    X[0] = 0.0                                       # zero vector
    X[1] *= 1e30                                     # huge
    X[2] *= 1e-30                                    # tiny
    X[3] = 0.0
    X[3, 17] = -2.5                                  # one-hot
    X[4] = 1.0                                       # constant
    X = synth.round_bf16(X)
    for bits in (1, 3):
        q = T.Quantizer(Rk, bits, variant, S if variant == "prod" else None, DEV)
        for dtype in ("bf16", "fp32"):
            p = T.encode(q, to_gpu_x(X, dtype))
            check_encode(gpu_packed_arrays(p, q), oracle_encode(X, Rk, S, bits, variant), bits, variant)


def test_encode_strided_and_tiny_batches(consts):
    Rk, _, S = consts
    g = np.random.default_rng(6)
    big = synth.round_bf16(g.standard_normal((40, 256)).astype(np.float32))
    q = T.Quantizer(Rk, 4, "prod", S, DEV)
    xt = to_gpu_x(big, "bf16")[:, 64:192]            # row stride 256 elements, offset 64
    for n in (1, 15, 16, 17, 40):
        p = T.encode(q, xt[:n])
        check_encode(gpu_packed_arrays(p, q), oracle_encode(big[:n, 64:192], Rk, S, 4, "prod"), 4, "prod")
    p = T.Packed(q, 0, DEV)
    T.encode(q, xt[:0], p)                           # n = 0 is a no-op
    torch.cuda.synchronize()


def test_encode_full_size_sampled(consts):
    # 2^20 tokens x 8 heads of bf16 Gaussian vectors, encoded in one call at the
    # size the benchmark times; 16384 rows sampled for the oracle.
    Rk, _, S = consts
    n = (1 << 20) * 8
    say("generating", n, "vectors")
    X = synth.gaussian((n, 128), 60, "bf16")
    xg = to_gpu_x(X, "bf16")
    rows = np.sort(np.random.default_rng(7).choice(n, 16384, replace=False))
    for bits, variant in ((3, "mse"), (4, "prod")):
        q = T.Quantizer(Rk, bits, variant, S if variant == "prod" else None, DEV)
        p = T.encode(q, xg)
        g = gpu_packed_arrays(p, q)
        say("full encode", bits, variant)
        check_encode({k: v[rows] for k, v in g.items()}, oracle_encode(X[rows], Rk, S, bits, variant),
                     bits, variant)


@pytest.mark.parametrize("variant,bits", [("mse", 4), ("prod", 4), ("mse", 2), ("prod", 3)])
def test_encode_close_thresholds(consts, variant, bits):
    """A codebook with two thresholds closer together than the encoder's cell
    table can separate (under 1.52/128 apart) makes the encoder keep its
    threshold search; the codes still follow idx = #{t_i < y} for that
    codebook, and the prod residual uses its centroids. Both table widths:
    3/4-bit and 2-bit searches."""
    Rk, _, S = consts
    bm = bits - 1 if variant == "prod" else bits
    c = book(bm)[0].astype(np.float32).astype(np.float64)
    h = len(c) // 2
    if bm >= 3:
        c[h + 1], c[h + 2] = c[h] + 0.002, c[h] + 0.004      # squeezed, still ascending
        c[h - 2], c[h - 3] = -c[h + 1], -c[h + 2]            # and antisymmetric
    else:
        c[h], c[h + 1] = 0.002, 0.004                        # thresholds -0.003, 0, 0.003
        c[h - 1], c[h - 2] = -c[h], -c[h + 1]
    t = (c[:-1] + c[1:]) / 2
    assert np.min(np.diff(t)) < 1.52 / 128
    q = T.Quantizer(Rk, bits, variant, S if variant == "prod" else None, DEV)
    q.centroids.copy_(torch.from_numpy(c.astype(np.float32)))
    q.boundaries[:len(t)].copy_(torch.from_numpy(t.astype(np.float32)))
    L.tq_prepare(q.c, None)
    n = 4096 + 37
    X = synth.outlier_kv(1, 1, n, 128, seed=120 + bm, dtype="bf16")[0, 0]
    say("encode close thresholds", variant, n)
    g = gpu_packed_arrays(T.encode(q, to_gpu_x(X, "bf16")), q)
    X64 = X.astype(np.float64)
    ref = encode_prod(X64, Rk, S, c, bits) if variant == "prod" else encode_mse(X64, Rk, c, bits)
    gidx = unpack_codes(g["codes"], 128, bm)
    mism = gidx != ref["idx"]
    dist = np.min(np.abs(ref["y"][..., None] - t), axis=-1)
    assert np.all(dist[mism] < 1e-6), "code mismatch away from a boundary"
    assert mism.sum() <= 1e-5 * mism.size
    assert np.any(gidx == h + 1)                          # the squeezed cell is used
    np.testing.assert_allclose(g["norms"], ref["norms"], rtol=1e-6)
    if variant == "prod":
        ok = ~mism.any(axis=1)
        bad = (unpack_signs(g["qjl"], 128) != unpack_signs(ref["qjl"], 128)) & ok[:, None]
        assert np.all(np.abs(ref["z"][bad]) < 1e-6), "sketch bit flipped away from zero"
        np.testing.assert_allclose(g["gammas"][ok], ref["gammas"][ok], rtol=1e-5, atol=1e-6)

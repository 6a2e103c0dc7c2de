"""Pins of the oracle's decode attention (softmax(K q/√d)·V per query head, as
"I Spent 31 Hours On The Math Behind Turboquant…" states it in section "KV
Cache: The problem") against a library routine and special cases. CPU only."""
import math

import numpy as np
import torch

import synth
from oracle import attention, decode_attention, dequant_mse, encode_mse, lloyd_max


def test_matches_torch_sdpa():
    g = np.random.default_rng(0)
    B, Hq, Hkv, T, d = 2, 8, 2, 300, 128
    q = g.standard_normal((B, Hq, d))
    K = g.standard_normal((B, Hkv, T, d)) * 2
    V = g.standard_normal((B, Hkv, T, d))
    out = decode_attention(q, K, V, 1 / math.sqrt(d))
    G = Hq // Hkv
    Kr = torch.from_numpy(np.repeat(K, G, axis=1))
    Vr = torch.from_numpy(np.repeat(V, G, axis=1))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, :, None, :], Kr, Vr).squeeze(2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_special_cases():
    g = np.random.default_rng(1)
    d, T = 128, 50
    K = g.standard_normal((T, d))
    V = g.standard_normal((T, d))
    # q = 0: uniform weights, the mean of the values
    np.testing.assert_allclose(attention(np.zeros(d), K, V, 0.1), V.mean(0), atol=1e-14)
    # one token: its value
    np.testing.assert_allclose(attention(g.standard_normal(d), K[:1], V[:1], 0.1), V[0], atol=0)
    # a dominant key takes all the weight
    q = K[7] * 100
    np.testing.assert_allclose(attention(q, K, V, 1.0), V[7], atol=1e-12)


def test_ctx_lens_and_gqa_map():
    g = np.random.default_rng(2)
    B, Hq, Hkv, T, d = 3, 6, 3, 40, 16
    q = g.standard_normal((B, Hq, d))
    K = g.standard_normal((B, Hkv, T, d))
    V = g.standard_normal((B, Hkv, T, d))
    lens = [40, 1, 17]
    out = decode_attention(q, K, V, 0.25, ctx_lens=lens)
    for b in range(B):
        for h in range(Hq):
            kv = h // 2
            s = K[b, kv, :lens[b]] @ q[b, h] * 0.25
            p = np.exp(s - s.max())
            np.testing.assert_allclose(out[b, h], p @ V[b, kv, :lens[b]] / p.sum(), atol=1e-13)


def test_rotated_space_identity():
    # The quantized cache can be attended in the rotated space: ⟨q, nΠᵀc⟩ =
    # n⟨Πq, c⟩ and Σ p n Πᵀc = Πᵀ(Σ p n c). Equal to the plain definition.
    d, T, b = 128, 256, 3
    c, _, _ = lloyd_max(d, b)
    R = synth.rotation(d, 9)
    g = np.random.default_rng(3)
    K = g.standard_normal((T, d))
    V = g.standard_normal((T, d))
    ek, ev = encode_mse(K, R, c, b), encode_mse(V, R, c, b)
    Kt = dequant_mse(ek["codes"], ek["norms"], R, c, b)
    Vt = dequant_mse(ev["codes"], ev["norms"], R, c, b)
    q = g.standard_normal(d)
    plain = attention(q, Kt, Vt, 1 / math.sqrt(d))
    Rd = R.astype(np.float64)
    s = ek["norms"] * (c[ek["idx"]] @ (Rd @ q)) / math.sqrt(d)
    p = np.exp(s - s.max())
    acc = (p * ev["norms"]) @ c[ev["idx"]]
    rot_form = Rd.T @ acc / p.sum()
    np.testing.assert_allclose(rot_form, plain, rtol=1e-12, atol=1e-13)

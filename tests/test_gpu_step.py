"""GPU tests of the decode step (tq_decode_step) and of the row-tile encoder
that small encodes and the step's appends use, through the C ABI:
  * the row-tile encoder gives bit-identical results to the full-size one;
  * the step equals tq_encode of the new rows into their slots followed by
    tq_attn_decode, bit for bit (caches and outputs), for ragged, empty and
    out-of-range lengths;
  * the step's appended rows and its output agree with the oracle."""
import math

import numpy as np
import pytest
import torch

import synth
from kv_cache_vector_06_amd import torch_api as T
from gpu_util import (DEV, assert_guards, check_encode, encode_away_from_ties, gpu_packed_arrays,
                      guarded_decoder, guarded_tensor, oracle_dequant, packed_from_oracle, quantizers,
                      rel_l2_per_head, say, to_gpu_x)
from oracle import decode_attention

pytestmark = pytest.mark.gpu
TOL = 1e-3
ROW_TILE_MAX_ROWS = 64 * 16      # encodes of at most this many rows take the row-tile form


def _rows(n, seed, dtype):
    """Seeded rows with a spread of magnitudes, a zero row and a huge row."""
    x = synth.gaussian((n, 128), seed, "fp32")
    x *= np.exp(np.random.default_rng(seed + 1).normal(0.0, 2.0, (n, 1))).astype(np.float32)
    x[3] = 0.0
    x[5] *= 1e30
    x[7] *= 1e-30
    return synth.round_bf16(x) if dtype == "bf16" else x


def _same_packed(a: T.Packed, b: T.Packed, rows=slice(None)):
    torch.cuda.synchronize()
    for name in ("codes", "norms", "qjl", "gammas"):
        x, y = getattr(a, name), getattr(b, name)
        if x is None:
            continue
        xa, ya = x[rows].cpu(), y[rows].cpu()
        if xa.dtype == torch.float32:
            xa, ya = xa.view(torch.int32), ya.view(torch.int32)
        assert torch.equal(xa, ya), name


@pytest.mark.parametrize("variant,bits", [("mse", 1), ("mse", 2), ("mse", 3), ("mse", 4),
                                          ("prod", 1), ("prod", 2), ("prod", 3), ("prod", 4)])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_row_tile_encoder_matches_full_size(variant, bits, dtype):
    say("row-tile encoder", variant, bits, dtype)
    Rk, _, S = synth.constants(128)
    q = T.Quantizer(Rk, bits, variant, S if variant == "prod" else None, DEV)
    n_big = 4096
    X = _rows(n_big, 900 + bits + (10 if variant == "prod" else 0), dtype)
    xg = to_gpu_x(X, dtype)
    big = T.encode(q, xg)                               # full-size encoder (256 tiles)
    for n in (1, 37, ROW_TILE_MAX_ROWS):
        small = T.encode(q, xg[:n])                     # row-tile encoder
        _same_packed(small, big, slice(0, n))
    # strided rows and scattered output slots
    wide = torch.zeros((50, 256), dtype=xg.dtype, device=DEV)
    wide[:, 64:192] = xg[:50]
    out = T.Packed(q, 200, DEV)
    slots = torch.arange(199, 99, -2, dtype=torch.int64, device=DEV)
    T.encode(q, wide[:, 64:192], out, slots)
    ref = T.Packed(q, 50, DEV)
    T.encode(q, xg[:50], ref)
    got, exp = gpu_packed_arrays(out, q), gpu_packed_arrays(ref, q)
    idx = slots.cpu().numpy()
    for k in exp:
        np.testing.assert_array_equal(got[k][idx], exp[k])


def _step_case(cfg, T_ctx, B, lens, dtype, seed):
    """Run the step and the unfused path (encode into slots, then decode) on
    identical caches; both must agree bit for bit."""
    say("step case", cfg.name, "T", T_ctx, "B", B, "lens", lens, dtype)
    kq, vq, Rk, Rv, S = quantizers(cfg)
    K, V = synth.make_kv(cfg, T=T_ctx, B=B)
    kp = T.encode(kq, to_gpu_x(K.reshape(-1, 128), cfg.dtype))
    vp = T.encode(vq, to_gpu_x(V.reshape(-1, 128), cfg.dtype))
    rows = B * cfg.Hkv
    kn = _rows(rows + 8, seed, dtype)[8:]
    vn = _rows(rows + 8, seed + 1, dtype)[8:]
    kng, vng = to_gpu_x(kn, dtype), to_gpu_x(vn, dtype)
    qg = torch.from_numpy(synth.make_query(cfg, B=B)).to(DEV)
    lg = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    dec = T.Decoder(B, cfg.Hq, cfg.Hkv, T_ctx, DEV)

    def clone(p, q):
        c = T.Packed(q, p.n, DEV)
        for name in ("codes", "norms", "qjl", "gammas"):
            if getattr(p, name) is not None:
                getattr(c, name).copy_(getattr(p, name))
        return c

    ka, va, kb, vb = clone(kp, kq), clone(vp, vq), clone(kp, kq), clone(vp, vq)
    # unfused: rows whose length is in [1, T] go to slot row*T + len - 1
    L = [T_ctx] * B if lens is None else lens
    sel = [b * cfg.Hkv + h for b in range(B) for h in range(cfg.Hkv) if 1 <= L[b] <= T_ctx]
    if sel:
        slots = torch.tensor([r * T_ctx + L[r // cfg.Hkv] - 1 for r in sel], dtype=torch.int64, device=DEV)
        idx = torch.tensor(sel, dtype=torch.int64, device=DEV)
        T.encode(kq, kng[idx].contiguous(), ka, slots)
        T.encode(vq, vng[idx].contiguous(), va, slots)
    out_a = dec(kq, vq, qg, ka, va, lg)
    out_b = dec.step(kq, vq, kng, vng, qg, kb, vb, lg)
    torch.cuda.synchronize()
    _same_packed(ka, kb)
    _same_packed(va, vb)
    assert torch.equal(out_a.view(torch.int32), out_b.view(torch.int32))
    return out_b


@pytest.mark.parametrize("name", synth.DECODE_WORKLOADS)
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_step_equals_append_then_decode(name, dtype):
    cfg = synth.WORKLOADS[name]
    B = min(cfg.B, 3)
    _step_case(cfg, 777, B, None, dtype, 40 + cfg.seed_base // 10)


def test_step_ragged_empty_and_out_of_range_lengths():
    cfg = synth.WORKLOADS["gqa8_prod4_128k_b4"]
    out = _step_case(cfg, 600, 5, [600, 1, 0, 333, 601], "bf16", 60)
    assert torch.all(out[2] == 0)
    cfg = synth.DecodeConfig("prod1_g3", 3, 2, 6, 300, 128, "prod", 1, 2, "lognormal", "fp32", 61)
    _step_case(cfg, 300, 3, [1, 300, 150], "fp32", 62)
    cfg = synth.DecodeConfig("gqa16", 2, 2, 32, 400, 128, "prod", 3, 3, "gaussian", "bf16", 63)
    _step_case(cfg, 400, 2, [399, 64], "bf16", 64)


def test_step_full_size():
    # The benchmark shape: 4 x 8 KV heads x 131072 tokens, 64 query heads.
    cfg = synth.WORKLOADS["gqa8_prod4_128k_b4"]
    kq, vq, Rk, Rv, S = quantizers(cfg)
    B, Tc = cfg.B, cfg.T
    say("full-size step: random packed caches")
    g = torch.Generator(device=DEV).manual_seed(5)
    kp, vp = T.Packed(kq, B * cfg.Hkv * Tc, DEV), T.Packed(vq, B * cfg.Hkv * Tc, DEV)
    for p in (kp, vp):
        p.codes.copy_(torch.randint(0, 256, p.codes.shape, dtype=torch.uint8, device=DEV, generator=g))
        p.norms.uniform_(0.5, 2.0, generator=g)
        if p.qjl is not None:
            p.qjl.copy_(torch.randint(0, 256, p.qjl.shape, dtype=torch.uint8, device=DEV, generator=g))
            p.gammas.uniform_(0.0, 0.5, generator=g)
    lens = [Tc, Tc - 1, 65536, 12345]
    lg = torch.tensor(lens, dtype=torch.int32, device=DEV)
    rows = B * cfg.Hkv
    kng = to_gpu_x(_rows(rows + 8, 70, "bf16")[8:], "bf16")
    vng = to_gpu_x(_rows(rows + 8, 71, "bf16")[8:], "bf16")
    qg = torch.from_numpy(synth.make_query(cfg)).to(DEV)
    dec = T.Decoder(B, cfg.Hq, cfg.Hkv, Tc, DEV)
    slots = torch.tensor([r * Tc + lens[r // cfg.Hkv] - 1 for r in range(rows)], dtype=torch.int64, device=DEV)
    kk, vv = T.Packed(kq, rows, DEV), T.Packed(vq, rows, DEV)
    T.encode(kq, kng, kk)
    T.encode(vq, vng, vv)
    out = dec.step(kq, vq, kng, vng, qg, kp, vp, lg)
    torch.cuda.synchronize()
    # appended rows equal the plain encode of the new rows
    for name in ("codes", "norms", "qjl", "gammas"):
        x = getattr(kp, name)[slots].cpu()
        y = getattr(kk, name).cpu()
        assert torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x,
                           y.view(torch.int32) if y.dtype == torch.float32 else y), name
    assert torch.equal(vp.codes[slots].cpu(), vv.codes.cpu())
    assert torch.equal(vp.norms[slots].cpu().view(torch.int32), vv.norms.cpu().view(torch.int32))
    # and the output equals a plain decode over the updated caches
    out2 = dec(kq, vq, qg, kp, vp, lg)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), out2.view(torch.int32))


def test_step_matches_oracle():
    # The oracle encodes every token (the last one of each row being the step's
    # new token) and evaluates attention; the GPU holds the oracle's cache for
    # the earlier tokens and appends the last one itself.
    cfg = synth.WORKLOADS["llama8b_prod3_128k"]
    B, Tc = 2, 900
    lens = [Tc, 500]
    kq, vq, Rk, Rv, S = quantizers(cfg)
    K, V = synth.make_kv(cfg, T=Tc, B=B)
    K, V = np.ascontiguousarray(K), np.ascontiguousarray(V)
    ek = encode_away_from_ties(K.reshape(-1, 128), Rk, S, cfg.k_bits, cfg.k_variant, 81, cfg.dtype)
    ev = encode_away_from_ties(V.reshape(-1, 128), Rv, None, cfg.v_bits, "mse", 82, cfg.dtype)
    shape = (B, cfg.Hkv, Tc, 128)
    Kt = oracle_dequant(ek, Rk, S, cfg.k_bits, cfg.k_variant).reshape(shape)
    Vt = oracle_dequant(ev, Rv, None, cfg.v_bits, "mse").reshape(shape)
    q = synth.make_query(cfg, B=B)
    ref = decode_attention(q, Kt, Vt, 1 / math.sqrt(128), ctx_lens=lens)
    # new rows: token lens[b] - 1 of each (b, KV head)
    new_idx = np.array([(b * cfg.Hkv + h) * Tc + lens[b] - 1 for b in range(B) for h in range(cfg.Hkv)])
    kn, vn = K.reshape(-1, 128)[new_idx], V.reshape(-1, 128)[new_idx]
    kp, vp = packed_from_oracle(ek, kq), packed_from_oracle(ev, vq)
    for p in (kp, vp):                                  # the step must write these slots
        sl = torch.from_numpy(new_idx).to(DEV)
        p.codes[sl] = 0
        p.norms[sl] = 0
        if p.qjl is not None:
            p.qjl[sl] = 0
            p.gammas[sl] = 0
    dec = guarded_decoder(B, cfg.Hq, cfg.Hkv, Tc)
    og, og_guard = guarded_tensor((B, cfg.Hq, 128), torch.float32)
    out = dec.step(kq, vq, to_gpu_x(kn, cfg.dtype), to_gpu_x(vn, cfg.dtype), torch.from_numpy(q).to(DEV),
                   kp, vp, torch.tensor(lens, dtype=torch.int32, device=DEV), out=og).cpu().numpy()
    assert_guards(dec, og_guard, kp, vp)
    gk, gv = gpu_packed_arrays(kp, kq), gpu_packed_arrays(vp, vq)
    sub = lambda e: {k: v[new_idx] for k, v in e.items()}
    ks = check_encode(sub(gk), sub(ek), cfg.k_bits, cfg.k_variant)
    vs = check_encode(sub(gv), sub(ev), cfg.v_bits, "mse")
    assert ks.get("code_mismatch", 0) == 0 and ks.get("sketch_mismatch", 0) == 0
    assert vs.get("code_mismatch", 0) == 0
    r = rel_l2_per_head(out, ref)
    say("  step vs oracle rel L2 max", r.max())
    assert r.max() <= TOL

#!/usr/bin/env python3
"""TurboQuant hot-path benchmark on one MI355X.

Workload: batch 4 x 8 KV heads x 131072 tokens, 64 query heads (GQA 8),
d = 128; keys TurboQuant-prod at 4 bits (3-bit Lloyd-Max + 1-bit QJL sketch),
values TurboQuant-mse at 4 bits; bf16 N(0,1) synthetic K/V (seeded). Plus the
prefill-scale encode sweep over 2^20 tokens x 8 heads.

One step = one pass of the whole hot path on resident inputs: encode the new
token's key and value of every (batch, KV head), append them to the packed
cache, then decode attention of every query head over the 131072-token packed
cache (tq_decode_step: the appends and the query operands in one launch, then
the split attention and the merge). Steps rotate over three
copies of the packed cache, so no step finds its cache in the 256 MB
last-level cache.

Prints one JSON line. `value` is packed-cache bytes read by decode per step /
step time (GB/s), timed without any event between the steps. `roofline` is
for the dominant kernel (the split-attention launch), timed with HIP events
around that launch on its stream in a second run of the same steps.
`hadamard_step_ms` / `hadamard_value` time the same step with randomized
Walsh-Hadamard rotations for keys and values; the encode sweep adds mse-4 and
prod-4 with that rotation. `search` times inner-product top-10 of 64 queries
over 2^20 prod-4 rows (with recall 1@10); `outlier_split` times encode and
decode of the 2.5- and 3.5-bit outlier-channel split caches at the same shape.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_F16_TFLOPS = 2500.0      # dense fp16 matrix cores
WORKLOAD = "gqa8_prod4_128k_b4"


def _src_hash(name: str) -> str:
    with open(os.path.join(ROOT, "kv_cache_vector_06_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic(kernel_file: str, src: str, launches_bytes: float):
    """HBM bytes per launch from committed rocprofv3 counter summaries, or None
    when absent or taken on another version of the kernel source."""
    path = os.path.join(ROOT, "profiles", kernel_file)
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha") != _src_hash(src):
        return None
    return rec.get("hbm_bytes_per_launch")


def _mfma_busy(kernel_row: str):
    """Matrix-core busy fraction of a kernel from the committed rocprofv3 SQ
    counter summary, or None when absent or taken on another encoder source."""
    path = os.path.join(ROOT, "profiles", "sq_counters_gqa8_prod4_128k.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        lines = f.read().splitlines()
    if not any(l.startswith("# src sha256") and f"tq_encode.hip {_src_hash('tq_encode.hip')}" in l for l in lines):
        return None
    for l in lines:
        if l.startswith(kernel_row):
            return float(l[len(kernel_row):].split()[5])
    return None


def cpu_baseline(cfg, units=6):
    """The oracle, as it stands, on a bounded sample of the same workload: the
    first `units` (batch, KV head) pairs of batch row 0, each encoded (keys and
    values over all 131072 tokens) and then decoded for its query heads."""
    import numpy as np
    import synth
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    Rk, Rv, S = synth.constants(cfg.d)
    T = cfg.T
    K, V = synth.make_kv(cfg, T=T, B=1)
    q = synth.make_query(cfg, B=1)[0].astype(np.float64)
    ck = oracle.lloyd_max(cfg.d, cfg.k_bits - 1)[0]
    cv = oracle.lloyd_max(cfg.d, cfg.v_bits)[0]
    chunk = 8192
    t_enc = t_dec = 0.0
    for h in range(units):
        Kx, Vx = K[0, h].astype(np.float64), V[0, h].astype(np.float64)
        t0 = time.perf_counter()
        ek = [oracle.encode_prod(Kx[i:i + chunk], Rk, S, ck, cfg.k_bits) for i in range(0, T, chunk)]
        ev = [oracle.encode_mse(Vx[i:i + chunk], Rv, cv, cfg.v_bits) for i in range(0, T, chunk)]
        t_enc += time.perf_counter() - t0
        t0 = time.perf_counter()
        Kt = np.concatenate([oracle.dequant_prod(e["codes"], e["norms"], e["qjl"], e["gammas"], Rk, S, ck,
                                                 cfg.k_bits) for e in ek])
        Vt = np.concatenate([oracle.dequant_mse(e["codes"], e["norms"], Rv, cv, cfg.v_bits) for e in ev])
        for hq in range(h * cfg.G, (h + 1) * cfg.G):
            oracle.attention(q[hq], Kt, Vt, 1 / math.sqrt(cfg.d))
        t_dec += time.perf_counter() - t0
    bytes_units = units * T * bytes_per_token(cfg)
    return {
        "value": round(bytes_units / t_dec / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": f"{units} of {cfg.B * cfg.Hkv} (batch, KV head) units, {T} tokens and {cfg.G} query heads "
                  f"each; decode = dequantize + softmax attention in float64",
        "decode_s": round(t_dec, 3),
        "encode_mvec_s": round(2 * units * T / t_enc / 1e6, 5), "encode_s": round(t_enc, 3),
        "encode_sample": f"{2 * units * T} vectors (keys prod-{cfg.k_bits}, values mse-{cfg.v_bits})",
        "host_cpus": os.cpu_count(),
    }


def _pct(sorted_vals, f: float) -> float:
    """The f-quantile of an ascending list (nearest rank)."""
    return sorted_vals[min(len(sorted_vals) - 1, max(0, round(f * (len(sorted_vals) - 1))))]


def key_bytes(cfg) -> int:
    """Packed bytes of one key vector: codes + fp32 norm, plus the 16-byte
    sketch and fp32 γ for prod keys."""
    d = cfg.d
    kb = cfg.k_bits - 1 if cfg.k_variant == "prod" else cfg.k_bits
    return d * kb // 8 + 4 + ((d // 8 + 4) if cfg.k_variant == "prod" else 0)


def bytes_per_token(cfg) -> int:
    """Algorithmic packed bytes per token per KV head: the key's, and the
    value's codes + fp32 norm."""
    return key_bytes(cfg) + cfg.d * cfg.v_bits // 8 + 4


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # Under sustained load the chip's clocks ramp up over the first ~200 steps
    # (≈30 ms) and fall back after idling; the warm-up covers the ramp, so the
    # timed steps measure the steady state.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-encode-sweep", action="store_true")
    ap.add_argument("--no-split", action="store_true", help="skip the outlier-channel split workloads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 512 MiB device copy (reference kernel for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this hot path runs on one GPU only (no multi-GPU path is built); "
              "use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    from kv_cache_vector_06_amd import torch_api as TA

    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    cfg = synth.WORKLOADS[WORKLOAD]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    B, Hkv, Hq, T, d = cfg.B, cfg.Hkv, cfg.Hq, cfg.T, cfg.d
    Rk, Rv, S = synth.constants(d)
    kq = TA.Quantizer(Rk, cfg.k_bits, cfg.k_variant, S, dev)
    vq = TA.Quantizer(Rv, cfg.v_bits, "mse", None, dev)

    log(f"[bench] generating {cfg.name}: B={B} Hkv={Hkv} T={T}")
    K, V = synth.make_kv(cfg)
    kg = torch.from_numpy(K.reshape(-1, d)).to(torch.bfloat16).to(dev)
    vg = torch.from_numpy(V.reshape(-1, d)).to(torch.bfloat16).to(dev)
    del K, V
    n_vec = B * Hkv * T
    # Three copies of the packed cache, used in turn: each step reads a cache
    # that two other steps' reads (1.2 GB) have since pushed out of the 256 MB
    # last-level cache, as when one layer's cache is read once per step.
    ncopy = 3
    kcs = [TA.Packed(kq, n_vec, dev) for _ in range(ncopy)]
    vcs = [TA.Packed(vq, n_vec, dev) for _ in range(ncopy)]
    TA.encode(kq, kg, kcs[0])
    TA.encode(vq, vg, vcs[0])
    for c in range(1, ncopy):
        for src, dst in ((kcs[0], kcs[c]), (vcs[0], vcs[c])):
            for name in ("codes", "norms", "qjl", "gammas"):
                if getattr(src, name) is not None:
                    getattr(dst, name).copy_(getattr(src, name))
    torch.cuda.synchronize()
    log("[bench] packed cache ready")

    q = torch.from_numpy(synth.make_query(cfg)).to(dev)
    g = np.random.default_rng(cfg.seed_base + 5)
    knew = torch.from_numpy(synth.round_bf16(g.standard_normal((B * Hkv, d)).astype(np.float32))).to(torch.bfloat16).to(dev)
    vnew = torch.from_numpy(synth.round_bf16(g.standard_normal((B * Hkv, d)).astype(np.float32))).to(torch.bfloat16).to(dev)
    dec = TA.Decoder(B, Hq, Hkv, T, dev)
    out = torch.empty_like(q)
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]

    def step(i, ev=None, qs=(kq, vq)):
        # tq_decode_step: the new token of every (batch, KV head) goes to slot
        # T - 1 (ctx_lens = NULL: every row is T long), then attention.
        kc, vc = kcs[i % ncopy], vcs[i % ncopy]
        if ev is None:
            dec.step(*qs, knew, vnew, q, kc, vc, out=out)
        else:
            dec.step(*qs, knew, vnew, q, kc, vc, out=out, phase=1)
            ev[0].record()
            dec.step(*qs, knew, vnew, q, kc, vc, out=out, phase=2)
            ev[1].record()
            dec.step(*qs, knew, vnew, q, kc, vc, out=out, phase=3)

    if args.copy_calibration:
        src = torch.empty(1 << 27, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)                # reads 512 MiB, writes 512 MiB
        torch.cuda.synchronize()
        del src, dst
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    # The dominant kernel: HIP events on its stream around its launch, in a
    # second run of the same steps (the events' own gaps stay out of the step
    # time above).
    for i in range(args.steps):
        step(i, (ev0[i], ev1[i]))
    torch.cuda.synchronize()
    k_ms = sorted(ev0[i].elapsed_time(ev1[i]) for i in range(args.steps))
    k_avg = sum(k_ms) / len(k_ms)
    # Spread of whole steps: one event after each step, in a third run (the
    # events add their own small gaps, so the median sits a little above the
    # event-free step time).
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record()
    for i in range(args.steps):
        step(i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    step_us = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(args.steps))
    bpt = bytes_per_token(cfg)
    dec_bytes = n_vec * bpt
    value = dec_bytes / (ms_step * 1e-3) / 1e9
    achieved = dec_bytes / (k_avg * 1e-3) / 1e9
    log(f"[bench] step {ms_step:.4f} ms; split-attention kernel avg {k_avg * 1e3:.1f} us "
        f"(min {k_ms[0] * 1e3:.1f}, max {k_ms[-1] * 1e3:.1f}); {achieved:.0f} GB/s")

    # Same kernel on one copy, right after reading 1 GiB elsewhere (clean
    # lines: nothing of the packed cache stays in the last-level cache and no
    # write-back competes with the launch).
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    fl = []
    for i in range(3):
        dec(kq, vq, q, kcs[0], vcs[0], out=out, phase=1)
        flush.sum()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        dec(kq, vq, q, kcs[0], vcs[0], out=out, phase=2)
        b_.record()
        torch.cuda.synchronize()
        fl.append(a_.elapsed_time(b_))
    flushed_us = sorted(fl)[len(fl) // 2] * 1e3
    log(f"[bench] split-attention after a read-only cache flush: median {flushed_us:.1f} us")

    # The part's practical read ceiling: one plain coalesced read
    # (tq_read_probe, the decode stream's 16-byte non-temporal loads) of as
    # many bytes as the packed cache, and of 4 GiB, back to back, each launch
    # timed by events around it. A read carries a fixed cost of its own (the
    # same-size read is the fair ceiling of one decode launch); the 4 GiB read
    # gives the rate with that cost spread thin.
    xo = torch.zeros(1, dtype=torch.int32, device=dev)
    big = torch.empty(1 << 30, dtype=torch.float32, device=dev).fill_(1.0)

    def read_us(buf):
        for _ in range(20):
            TA.read_probe(buf, xo)
        pr = []
        for _ in range(30):
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record()
            TA.read_probe(buf, xo)
            b_.record()
            pr.append((a_, b_))
        torch.cuda.synchronize()
        return sorted(a_.elapsed_time(b_) for a_, b_ in pr)[len(pr) // 2] * 1e3

    pr_us = read_us(flush.view(torch.uint8)[:dec_bytes])
    read_peak = dec_bytes / (pr_us * 1e-6) / 1e9
    pr4_us = read_us(big)
    read_peak_4g = big.numel() * 4 / (pr4_us * 1e-6) / 1e9
    del flush, xo, big
    log(f"[bench] plain read of {dec_bytes} B: median {pr_us:.1f} us, {read_peak:.0f} GB/s; "
        f"of 4 GiB: {pr4_us:.1f} us, {read_peak_4g:.0f} GB/s")

    # The same step with randomized Walsh-Hadamard rotations for keys and
    # values (the caches re-encoded with them).
    Rkh, Rvh, _ = synth.hadamard_constants(d)
    kqh = TA.Quantizer(Rkh, cfg.k_bits, cfg.k_variant, S, dev, "hadamard")
    vqh = TA.Quantizer(Rvh, cfg.v_bits, "mse", None, dev, "hadamard")
    for c in range(ncopy):
        TA.encode(kqh, kg, kcs[c])
        TA.encode(vqh, vg, vcs[c])
    for i in range(args.warmup):
        step(i, qs=(kqh, vqh))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, qs=(kqh, vqh))
    torch.cuda.synchronize()
    had_ms = (time.perf_counter() - t0) / args.steps * 1e3
    log(f"[bench] step with Hadamard rotations {had_ms:.4f} ms")

    # The other 128K workload: batch 1, 8 KV heads, 32 query heads, prod-3 keys,
    # mse-3 values (113 MB packed, which fits the 256 MB last-level cache: the
    # split launch is timed alone, after a 1 GiB read).
    del kcs, vcs
    torch.cuda.empty_cache()
    cfg_b1 = synth.WORKLOADS["llama8b_prod3_128k"]
    kq3 = TA.Quantizer(Rk, cfg_b1.k_bits, cfg_b1.k_variant, S, dev)
    vq3 = TA.Quantizer(Rv, cfg_b1.v_bits, "mse", None, dev)
    K3, V3 = synth.make_kv(cfg_b1)
    n3 = cfg_b1.B * cfg_b1.Hkv * cfg_b1.T
    kc3, vc3 = TA.Packed(kq3, n3, dev), TA.Packed(vq3, n3, dev)
    TA.encode(kq3, torch.from_numpy(K3.reshape(-1, d)).to(torch.bfloat16).to(dev), kc3)
    TA.encode(vq3, torch.from_numpy(V3.reshape(-1, d)).to(torch.bfloat16).to(dev), vc3)
    del K3, V3
    q3 = torch.from_numpy(synth.make_query(cfg_b1)).to(dev)
    dec3 = TA.Decoder(cfg_b1.B, cfg_b1.Hq, cfg_b1.Hkv, cfg_b1.T, dev)
    out3 = torch.empty_like(q3)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    fl3 = []
    for i in range(7):
        dec3(kq3, vq3, q3, kc3, vc3, out=out3, phase=1)
        flush.sum()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        dec3(kq3, vq3, q3, kc3, vc3, out=out3, phase=2)
        b_.record()
        torch.cuda.synchronize()
        fl3.append(a_.elapsed_time(b_))
    cfg_b1_us = sorted(fl3)[len(fl3) // 2] * 1e3
    cfg_b1_bytes = n3 * bytes_per_token(cfg_b1)
    # Its ceiling: a plain read (tq_read_probe) of as many bytes, also after
    # a 1 GiB read, so that none of them is in the last-level cache.
    rb = torch.ones(cfg_b1_bytes // 4, dtype=torch.float32, device=dev)
    xo3 = torch.zeros(1, dtype=torch.int32, device=dev)
    rd3 = []
    for i in range(7):
        flush.sum()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        TA.read_probe(rb, xo3)
        b_.record()
        torch.cuda.synchronize()
        rd3.append(a_.elapsed_time(b_))
    del flush, kc3, vc3, rb, xo3
    cfg_b1_read_us = sorted(rd3)[len(rd3) // 2] * 1e3
    log(f"[bench] {cfg_b1.name}: split attention after a cache flush {cfg_b1_us:.1f} us, "
        f"{cfg_b1_bytes / cfg_b1_us / 1e3:.0f} GB/s; plain read of as many bytes {cfg_b1_read_us:.1f} us")

    # Inner-product search: the first 2^20 key rows as a prod-4 database
    # (index build = their encode), 64 N(0,1) queries, top 10 each; recall 1@10
    # against the exact top-1 of the unquantized rows.
    n_db, nq_s, k_s = 1 << 20, 64, 10
    db = TA.Packed(kq, n_db, dev)
    a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    TA.encode(kq, kg[:n_db], db)
    a_.record()
    TA.encode(kq, kg[:n_db], db)
    b_.record()
    torch.cuda.synchronize()
    build_ms = a_.elapsed_time(b_)
    qs_ = torch.from_numpy(np.random.default_rng(cfg.seed_base + 7).standard_normal((nq_s, d)).astype(np.float32)).to(dev)
    ws_s = torch.empty(TA.L.tq_search_workspace(nq_s, n_db, k_s), dtype=torch.uint8, device=dev)
    for _ in range(3):
        TA.search(kq, qs_, db, k_s, workspace=ws_s)
    reps = 20
    a_.record()
    for _ in range(reps):
        _, s_idx = TA.search(kq, qs_, db, k_s, workspace=ws_s)
    b_.record()
    torch.cuda.synchronize()
    s_us = a_.elapsed_time(b_) / reps * 1e3
    top1 = (qs_ @ kg[:n_db].float().T).argmax(dim=1)
    recall = float((s_idx == top1[:, None]).any(dim=1).float().mean())
    db_bytes = n_db * key_bytes(cfg)
    search = {"workload": f"db {n_db} x d{d} prod-{cfg.k_bits}, {nq_s} queries, top {k_s}",
              "us": round(s_us, 1), "gpairs_s": round(nq_s * n_db / (s_us * 1e-6) / 1e9, 1),
              "db_gbs": round(db_bytes / (s_us * 1e-6) / 1e9, 1),
              "db_streamed_gbs": round((nq_s + 7) // 8 * db_bytes / (s_us * 1e-6) / 1e9, 1),
              "recall_1_at_10": round(recall, 4), "index_build_ms": round(build_ms, 4)}
    del ws_s
    log(f"[bench] search: {search}")

    # Outlier-channel split workloads ("2.5-bit": 32 channels at 3 bits + 96 at
    # 2, and "3.5-bit": 4 + 3; mse keys and values, a norm per group) at the
    # benchmark's shape: encode of the key cache, the decode call (query
    # operands, split attention, merge) over three cache copies in turn, and
    # the split-attention launch alone after a 1 GiB read.
    split_res = {}
    if not args.no_split:
        del db
        torch.cuda.empty_cache()
        for sname in ("gqa8_split25_128k_b4", "gqa8_split35_128k_b4"):
            cs = synth.WORKLOADS[sname]
            sc = synth.split_constants(d)
            kq6 = TA.Quantizer(None, cs.k_bits, "mse", None, dev, split=(sc["rk_o"], sc["rk_r"], sc["ch_k"]))
            vq6 = TA.Quantizer(None, cs.v_bits, "mse", None, dev, split=(sc["rv_o"], sc["rv_r"], sc["ch_v"]))
            K6, V6 = synth.make_kv(cs)
            k6 = torch.from_numpy(K6.reshape(-1, d)).to(torch.bfloat16).to(dev)
            v6 = torch.from_numpy(V6.reshape(-1, d)).to(torch.bfloat16).to(dev)
            del K6, V6
            n6 = cs.B * cs.Hkv * cs.T
            kc6 = [TA.Packed(kq6, n6, dev) for _ in range(ncopy)]
            vc6 = [TA.Packed(vq6, n6, dev) for _ in range(ncopy)]
            for c in range(ncopy):
                TA.encode(kq6, k6, kc6[c])
                TA.encode(vq6, v6, vc6[c])
            a_.record()
            TA.encode(kq6, k6, kc6[0])
            b_.record()
            torch.cuda.synchronize()
            enc6_ms = a_.elapsed_time(b_)
            del k6, v6
            dec6 = TA.Decoder(cs.B, cs.Hq, cs.Hkv, cs.T, dev)
            for i in range(args.warmup):
                dec6(kq6, vq6, q, kc6[i % ncopy], vc6[i % ncopy], out=out)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(args.steps):
                dec6(kq6, vq6, q, kc6[i % ncopy], vc6[i % ncopy], out=out)
            torch.cuda.synchronize()
            ms6 = (time.perf_counter() - t0) / args.steps * 1e3
            flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
            fl6 = []
            for i in range(5):
                dec6(kq6, vq6, q, kc6[0], vc6[0], out=out, phase=1)
                flush.sum()
                a_.record()
                dec6(kq6, vq6, q, kc6[0], vc6[0], out=out, phase=2)
                b_.record()
                torch.cuda.synchronize()
                fl6.append(a_.elapsed_time(b_))
            del flush, kc6, vc6
            torch.cuda.empty_cache()
            us6 = sorted(fl6)[len(fl6) // 2] * 1e3
            by6 = n6 * (kq6.code_bytes + 8 + vq6.code_bytes + 8)
            split_res[cs.name] = {
                "bytes_per_token_head": kq6.code_bytes + 8 + vq6.code_bytes + 8, "packed_cache_bytes": by6,
                "decode_ms": round(ms6, 5), "decode_gbs": round(by6 / (ms6 * 1e-3) / 1e9, 1),
                "split_after_flush_us": round(us6, 2), "split_gbs": round(by6 / us6 / 1e3, 1),
                "frac": round(by6 / us6 / 1e3 / PEAK_HBM_GBS, 4),
                "encode_mvec_s": round(n6 / (enc6_ms * 1e-3) / 1e6, 1)}
            log(f"[bench] {cs.name}: {split_res[cs.name]}")

    enc = {}
    enc_roof = None
    enc_mfma = {}
    if not args.no_encode_sweep:
        n_sweep = (1 << 20) * 8
        xs = torch.cat([kg, vg])[:n_sweep]
        for label, bits, var, rot in (("mse1", 1, "mse", "dense"), ("mse2", 2, "mse", "dense"),
                                      ("mse3", 3, "mse", "dense"), ("mse4", 4, "mse", "dense"),
                                      ("prod4", 4, "prod", "dense"), ("mse4_hadamard", 4, "mse", "hadamard"),
                                      ("prod4_hadamard", 4, "prod", "hadamard")):
            qq = TA.Quantizer(Rk if rot == "dense" else Rkh, bits, var, S if var == "prod" else None, dev, rot)
            pk = TA.Packed(qq, n_sweep, dev)
            TA.encode(qq, xs, pk)
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 3
            a_.record()
            for _ in range(reps):
                TA.encode(qq, xs, pk)
            b_.record()
            torch.cuda.synchronize()
            ms = a_.elapsed_time(b_) / reps
            enc[label] = round(n_sweep / (ms * 1e-3) / 1e6, 1)
            if label == "mse4":
                eb = n_sweep * (2 * d + d * 4 // 8 + 4)
                enc_roof = {"kernel": "encode_kernel<4,mse,bf16>", "bound": "hbm",
                            "achieved": round(eb / (ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(eb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                            "traffic": _traffic("encode_mse4_sweep.counters.json", "tq_encode.hip", eb)}
            if label in ("mse4", "prod4"):
                # Matrix-core use: the algorithmic flops (2d² per vector for the
                # rotation, 2d² more for the prod sketch) and the flops the
                # fp16 matrix cores execute with the operands split into hi/lo
                # parts (rotation 2 passes, sketch 3), against the dense fp16
                # peak; plus the busy fraction the SQ counters measured.
                alg = 2 * d * d * (2 if var == "prod" else 1)
                exe = 2 * d * d * (5 if var == "prod" else 2)
                rate = n_sweep / (ms * 1e-3)
                enc_mfma[label] = {"flops_per_vec": alg, "executed_flops_per_vec": exe,
                                   "tflops": round(rate * alg / 1e12, 1),
                                   "executed_tflops": round(rate * exe / 1e12, 1), "peak_tflops": PEAK_F16_TFLOPS,
                                   "frac": round(rate * alg / 1e12 / PEAK_F16_TFLOPS, 4),
                                   "executed_frac": round(rate * exe / 1e12 / PEAK_F16_TFLOPS, 4),
                                   "busy_counter": _mfma_busy(f"tq::encode_kernel<{bits - (var == 'prod')}, "
                                                              f"{'true' if var == 'prod' else 'false'}, false>")}
            del pk, qq
            log(f"[bench] encode {label}: {enc[label]} Mvec/s")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host")
        cpu = cpu_baseline(cfg)

    rec = {
        "metric": "packed-KV decode-attn HBM GB/s (% of peak) @128K ctx; encode Mvec/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16-mfma/f32",
        "data": "synthetic (seeded bf16 N(0,1) K/V, fp32 N(0,1) queries)",
        "config": {"workload": cfg.name, "B": B, "Hkv": Hkv, "Hq": Hq, "ctx": T, "d": d,
                   "keys": f"prod-{cfg.k_bits}", "values": f"mse-{cfg.v_bits}",
                   "step": "append 1 token per (batch, KV head) + decode all query heads",
                   "packed_bytes_per_token_head": bpt, "packed_cache_bytes": dec_bytes},
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "roofline": {"kernel": "attn_split_kernel<3,prod,4>", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": _traffic("attn_split_gqa8_prod4_128k.counters.json", "tq_decode.hip", dec_bytes),
                     "avg_launch_us": round(k_avg * 1e3, 2), "after_read_flush_us": round(flushed_us, 2),
                     "launch_us_p10_p50_p90": [round(_pct(k_ms, f) * 1e3, 2) for f in (0.1, 0.5, 0.9)],
                     "frac_of_measured_read": round(achieved / read_peak, 4),
                     "cache_copies": ncopy},
        "step_us_p10_p50_p90": [round(_pct(step_us, f), 2) for f in (0.1, 0.5, 0.9)],
        "measured_read_peak": {"gbs": round(read_peak, 1), "bytes": dec_bytes, "us": round(pr_us, 2),
                               "gbs_4gib": round(read_peak_4g, 1),
                               "kernel": "tq_read_probe: plain coalesced read, 16-byte non-temporal loads",
                               "value_frac": round(value / read_peak, 4)},
        "cfg_llama8b_prod3_128k": {"workload": cfg_b1.name, "packed_cache_bytes": cfg_b1_bytes,
                                   "split_after_flush_us": round(cfg_b1_us, 2),
                                   "split_gbs": round(cfg_b1_bytes / cfg_b1_us / 1e3, 1),
                                   "frac": round(cfg_b1_bytes / cfg_b1_us / 1e3 / PEAK_HBM_GBS, 4),
                                   "same_size_read_us": round(cfg_b1_read_us, 2),
                                   "frac_of_measured_read": round(cfg_b1_read_us / cfg_b1_us, 4)},
        "hadamard_step_ms": round(had_ms, 5),
        "hadamard_value": round(dec_bytes / (had_ms * 1e-3) / 1e9, 1),
        "search": search,
        "outlier_split": split_res,
        "encode_mvec_s": enc,
        "encode_roofline": enc_roof,
        "encode_mfma": enc_mfma or None,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""TurboQuant hot-path benchmark on one MI355X.

Headline workload (gqa8_prod4_128k_b4): batch 4 x 8 KV heads x 131072
tokens, 64 query heads (GQA 8), d = 128; keys TurboQuant-prod at 4 bits
(3-bit Lloyd-Max + 1-bit QJL sketch), values TurboQuant-mse at 4 bits; bf16
N(0,1) synthetic K/V (seeded).

One step = one pass of the whole hot path on resident inputs: encode the new
token's key and value of every (batch, KV head), append them to the packed
cache, then decode attention of every query head over the 131072-token packed
cache (tq_decode_step: the appends and the query operands in one launch, then
the split attention and the merge). Steps rotate over three copies of the
packed cache, so no step finds its cache in the 256 MB last-level cache.

Prints one JSON line.
  * `value`: packed-cache bytes read by decode per step / step time (GB/s),
    over `--steps` steps after `--warmup` untimed ones, right after the encode
    sweep (prefill-scale encode, then decode steps). In every timed step
    a pair of HIP events brackets the split-attention launch on its stream;
    `roofline` is that kernel's average over the same steps (so it can never
    exceed the step).
  * `steady_state`: the same step after 300 warm-up steps (the chip's clocks
    settle under sustained load over the first ~200 steps), 200 timed steps.
  * `configs`: the other workloads, each as decode steps back to back over
    rotating cache copies (enough to exceed the last-level cache where the
    cache is small), its split launch alone after a 1 GiB read, and a plain
    read (tq_read_probe) of as many bytes under the same conditions.
  * `encode_mvec_s` (+ `encode_roofline`, `encode_mfma`): the 2^20 x 8-vector
    bf16 encode sweep at mse-1..4 and prod-4 (dense and Hadamard rotations).
  * `search`, `outlier_split`, `hadamard_*`: the other built rows.
  * `cpu_baseline`: the float64 oracle on the host, one thread and all cores.
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
STEADY_WARMUP, STEADY_STEPS = 300, 200


def _src_hash(name: str) -> str:
    with open(os.path.join(ROOT, "kv_cache_vector_06_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic(kernel_file: str, src: str):
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


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_run(cfg, K, V, q, units):
    """Oracle encode (keys prod, values mse, full length) and decode of the
    first `units` (batch 0, KV head) pairs; returns (encode s, decode s)."""
    import numpy as np
    import synth
    import oracle
    Rk, Rv, S = synth.constants(cfg.d)
    T = cfg.T
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
    return t_enc, t_dec


def cpu_baseline(cfg):
    """The oracle, as it stands, on a bounded sample of the headline workload:
    whole (batch 0, KV head) units, each encoded (keys and values over all
    131072 tokens) and then decoded for its 8 query heads, in float64 numpy.
    Two modes: one thread (BLAS limited to 1) on 1 unit, and all host cores
    (BLAS threads) on 4 units."""
    import numpy as np
    import synth
    from threadpoolctl import threadpool_info, threadpool_limits

    K, V = synth.make_kv(cfg, T=cfg.T, B=1)
    K, V = K[:, :4], V[:, :4]
    q = synth.make_query(cfg, B=1)[0].astype(np.float64)
    bpt = bytes_per_token(cfg)
    res = {}
    for mode, units, limit in (("single_thread", 1, 1), ("all_cores", 4, None)):
        if limit is None:
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
            te, td = _oracle_run(cfg, K, V, q, units)
        else:
            with threadpool_limits(limits=limit):
                threads = limit
                te, td = _oracle_run(cfg, K, V, q, units)
        res[mode] = {"threads": threads, "units": units, "decode_gbs": round(units * cfg.T * bpt / td / 1e9, 5),
                     "decode_s": round(td, 3), "encode_mvec_s": round(2 * units * cfg.T / te / 1e6, 5),
                     "encode_s": round(te, 3)}
    allc = res["all_cores"]
    return {
        "value": allc["decode_gbs"], "unit": "GB/s", "cores": allc["threads"], "kind": "oracle",
        "sample": f"(batch 0, KV head) units of {cfg.name}, {cfg.T} tokens and {cfg.G} query heads each: "
                  f"encode = prod-{cfg.k_bits} keys + mse-{cfg.v_bits} values, decode = dequantize + softmax "
                  f"attention, float64 numpy; 1 unit single-threaded, 4 units on all cores",
        "single_thread": res["single_thread"], "all_cores": allc,
        "nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": _cpu_model(),
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
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-encode-sweep", action="store_true")
    ap.add_argument("--no-split", action="store_true", help="skip the outlier-channel split workloads")
    ap.add_argument("--no-configs", action="store_true", help="skip the other decode workloads")
    ap.add_argument("--quick", action="store_true",
                    help="the encode sweep and the headline steps only (for profiler runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 512 MiB device copy (reference kernel for HBM byte counters)")
    args = ap.parse_args()
    if args.quick:
        args.no_cpu_baseline = args.no_split = args.no_configs = True
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
    Event = lambda: torch.cuda.Event(enable_timing=True)

    log(f"[bench] generating {cfg.name}: B={B} Hkv={Hkv} T={T}")
    K, V = synth.make_kv(cfg)
    kg = torch.from_numpy(K.reshape(-1, d)).to(torch.bfloat16).to(dev)
    vg = torch.from_numpy(V.reshape(-1, d)).to(torch.bfloat16).to(dev)
    del K, V
    n_vec = B * Hkv * T

    def packed_copies(kq_, vq_, kx, vx, n, ncopy):
        """Encode kx/vx once, then copy the packed arrays into ncopy caches."""
        kcs = [TA.Packed(kq_, n, dev) for _ in range(ncopy)]
        vcs = [TA.Packed(vq_, n, dev) for _ in range(ncopy)]
        TA.encode(kq_, kx, kcs[0])
        TA.encode(vq_, vx, vcs[0])
        for c in range(1, ncopy):
            for src, dst in ((kcs[0], kcs[c]), (vcs[0], vcs[c])):
                for name in ("codes", "norms", "qjl", "gammas"):
                    if getattr(src, name) is not None:
                        getattr(dst, name).copy_(getattr(src, name))
        torch.cuda.synchronize()
        return kcs, vcs

    # Three copies of the packed cache, used in turn: each step reads a cache
    # that two other steps' reads (1.2 GB) have since pushed out of the 256 MB
    # last-level cache, as when one layer's cache is read once per step.
    ncopy = 3
    kcs, vcs = packed_copies(kq, vq, kg, vg, n_vec, ncopy)
    log("[bench] packed cache ready")

    q = torch.from_numpy(synth.make_query(cfg)).to(dev)
    g = np.random.default_rng(cfg.seed_base + 5)
    knew = torch.from_numpy(synth.round_bf16(g.standard_normal((B * Hkv, d)).astype(np.float32))).to(torch.bfloat16).to(dev)
    vnew = torch.from_numpy(synth.round_bf16(g.standard_normal((B * Hkv, d)).astype(np.float32))).to(torch.bfloat16).to(dev)
    dec = TA.Decoder(B, Hq, Hkv, T, dev)
    out = torch.empty_like(q)

    def timed_steps(dec_, qs, kcs_, vcs_, kn, vn, q_, out_, warmup, steps):
        """`warmup` untimed fused decode steps, then `steps` timed ones over the
        rotating cache copies, each with a pair of events around its split
        launch (phase 2) on the current stream. Returns (ms per step by the
        host clock between two synchronizations, split-launch µs list)."""
        nc = len(kcs_)
        for i in range(warmup):
            dec_.step(*qs, kn, vn, q_, kcs_[i % nc], vcs_[i % nc], out=out_)
        ea = [Event() for _ in range(steps)]
        eb = [Event() for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            kc, vc = kcs_[i % nc], vcs_[i % nc]
            dec_.step(*qs, kn, vn, q_, kc, vc, out=out_, phase=1)
            ea[i].record()
            dec_.step(*qs, kn, vn, q_, kc, vc, out=out_, phase=2)
            eb[i].record()
            dec_.step(*qs, kn, vn, q_, kc, vc, out=out_, phase=3)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / steps * 1e3
        return ms, [a.elapsed_time(b) * 1e3 for a, b in zip(ea, eb)]

    if args.copy_calibration:
        src = torch.empty(1 << 27, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)                # reads 512 MiB, writes 512 MiB
        torch.cuda.synchronize()
        del src, dst

    # ---- encode sweep (prefill-scale encode), right before the headline decode:
    # as in serving, where a prompt's keys and values are encoded and decode
    # steps follow, the chip is already under load when the decode steps start.
    # The quantizers and outputs are made first; then every configuration's
    # encodes run back to back (one untimed, then three between a pair of
    # events), with a single synchronization at the end.
    Rkh, Rvh, _ = synth.hadamard_constants(d)
    enc = {}
    enc_roof = enc_roof_prod = None
    enc_mfma = {}
    if not args.no_encode_sweep:
        n_sweep = (1 << 20) * 8
        xs = torch.cat([kg, vg])[:n_sweep]
        sweep = []
        for label, bits, var, rot in (("mse1", 1, "mse", "dense"), ("mse2", 2, "mse", "dense"),
                                      ("mse3", 3, "mse", "dense"), ("mse4", 4, "mse", "dense"),
                                      ("prod4", 4, "prod", "dense"), ("mse4_hadamard", 4, "mse", "hadamard"),
                                      ("prod4_hadamard", 4, "prod", "hadamard")):
            qq = TA.Quantizer(Rk if rot == "dense" else Rkh, bits, var, S if var == "prod" else None, dev, rot)
            sweep.append((label, bits, var, qq, TA.Packed(qq, n_sweep, dev), Event(), Event()))
        torch.cuda.synchronize()
        reps = 3
        for label, bits, var, qq, pk, a_, b_ in sweep:
            TA.encode(qq, xs, pk)
            a_.record()
            for _ in range(reps):
                TA.encode(qq, xs, pk)
            b_.record()
        torch.cuda.synchronize()
        for label, bits, var, qq, pk, a_, b_ in sweep:
            ms = a_.elapsed_time(b_) / reps
            enc[label] = round(n_sweep / (ms * 1e-3) / 1e6, 1)
            bm = bits - (var == "prod")
            eb = n_sweep * (2 * d + d * bm // 8 + 4 + ((d // 8 + 4) if var == "prod" else 0))
            if label in ("mse4", "prod4"):
                roof = {"kernel": f"encode_kernel<{bm},{var},bf16>", "bound": "hbm",
                        "achieved": round(eb / (ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(eb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
                if label == "mse4":
                    roof["traffic"] = _traffic("encode_mse4_sweep.counters.json", "tq_encode.hip")
                    enc_roof = roof
                else:
                    enc_roof_prod = roof
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
                                   "busy_counter": _mfma_busy(f"tq::encode_kernel<{bm}, "
                                                              f"{'true' if var == 'prod' else 'false'}, false>")}
            log(f"[bench] encode {label}: {enc[label]} Mvec/s")
        if enc_roof is not None and enc_roof_prod is not None:
            enc_roof["prod4"] = enc_roof_prod

    # ---- headline: the driver's warm-up and step counts ---------------------
    ms_step, k_us = timed_steps(dec, (kq, vq), kcs, vcs, knew, vnew, q, out, args.warmup, args.steps)
    k_avg = sum(k_us) / len(k_us)
    k_sorted = sorted(k_us)
    if k_avg > ms_step * 1e3:
        log(f"[bench] WARNING: split-launch average {k_avg:.1f} us exceeds the step {ms_step * 1e3:.1f} us")
    bpt = bytes_per_token(cfg)
    dec_bytes = n_vec * bpt
    value = dec_bytes / (ms_step * 1e-3) / 1e9
    achieved = dec_bytes / (k_avg * 1e-6) / 1e9
    log(f"[bench] step {ms_step:.4f} ms; split-attention kernel avg {k_avg:.1f} us "
        f"(min {k_sorted[0]:.1f}, max {k_sorted[-1]:.1f}); {achieved:.0f} GB/s")

    if not args.no_encode_sweep:
        del sweep, xs
        torch.cuda.empty_cache()

    # ---- the same step in the steady state -----------------------------------
    st_ms, st_k = timed_steps(dec, (kq, vq), kcs, vcs, knew, vnew, q, out, STEADY_WARMUP, STEADY_STEPS)
    st_kavg = sum(st_k) / len(st_k)
    steady = {"warmup": STEADY_WARMUP, "steps": STEADY_STEPS, "ms_per_step": round(st_ms, 5),
              "value": round(dec_bytes / (st_ms * 1e-3) / 1e9, 1),
              "frac": round(dec_bytes / (st_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
              "split_launch_us": round(st_kavg, 2),
              "split_gbs": round(dec_bytes / (st_kavg * 1e-6) / 1e9, 1),
              "split_frac": round(dec_bytes / (st_kavg * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
              "split_us_p10_p50_p90": [round(_pct(sorted(st_k), f), 2) for f in (0.1, 0.5, 0.9)]}
    log(f"[bench] steady state: {steady}")

    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)

    def flushed_split_us(dec_, kq_, vq_, q_, kc, vc, out_, reps):
        """Median µs of the split launch alone, each after a 1 GiB read (clean
        lines: nothing of the packed cache stays in the last-level cache)."""
        fl = []
        for _ in range(reps):
            dec_(kq_, vq_, q_, kc, vc, out=out_, phase=1)
            flush.sum()
            a_, b_ = Event(), Event()
            a_.record()
            dec_(kq_, vq_, q_, kc, vc, out=out_, phase=2)
            b_.record()
            torch.cuda.synchronize()
            fl.append(a_.elapsed_time(b_) * 1e3)
        return sorted(fl)[len(fl) // 2]

    flushed_us = flushed_split_us(dec, kq, vq, q, kcs[0], vcs[0], out, 3)
    log(f"[bench] split-attention after a read-only cache flush: median {flushed_us:.1f} us")

    # ---- read ceilings --------------------------------------------------------
    xo = torch.zeros(1, dtype=torch.int32, device=dev)

    def read_back_to_back_us(bufs, reps=30, warm=20):
        """Median µs of tq_read_probe over rotating buffers, back to back, each
        launch between a pair of events."""
        for i in range(warm):
            TA.read_probe(bufs[i % len(bufs)], xo)
        pr = []
        for i in range(reps):
            a_, b_ = Event(), Event()
            a_.record()
            TA.read_probe(bufs[i % len(bufs)], xo)
            b_.record()
            pr.append((a_, b_))
        torch.cuda.synchronize()
        return sorted(a_.elapsed_time(b_) for a_, b_ in pr)[len(pr) // 2] * 1e3

    def read_after_flush_us(buf, reps=7):
        rd = []
        for _ in range(reps):
            flush.sum()
            a_, b_ = Event(), Event()
            a_.record()
            TA.read_probe(buf, xo)
            b_.record()
            torch.cuda.synchronize()
            rd.append(a_.elapsed_time(b_) * 1e3)
        return sorted(rd)[len(rd) // 2]

    big = torch.empty(1 << 30, dtype=torch.float32, device=dev).fill_(1.0)
    pr_us = read_back_to_back_us([big.view(torch.uint8)[:dec_bytes]])
    read_peak = dec_bytes / (pr_us * 1e-6) / 1e9
    pr4_us = read_back_to_back_us([big])
    read_peak_4g = big.numel() * 4 / (pr4_us * 1e-6) / 1e9
    # Read time against size (every size above the 256 MB last-level cache, so
    # back-to-back reads of one buffer come from HBM): the least-squares line
    # t = t0 + bytes / bw splits a launch into a fixed part and a streaming part.
    sweep_mib = (512, 768, 1024, 1536, 2048, 3072, 4096)
    sweep_us = [read_back_to_back_us([big.view(torch.uint8)[:m << 20]], reps=20, warm=5) for m in sweep_mib]
    xs_b = [float(m << 20) for m in sweep_mib]
    mx, my = sum(xs_b) / len(xs_b), sum(sweep_us) / len(sweep_us)
    slope = sum((x - mx) * (y - my) for x, y in zip(xs_b, sweep_us)) / sum((x - mx) ** 2 for x in xs_b)
    read_sweep = {"mib": list(sweep_mib), "us": [round(u, 2) for u in sweep_us],
                  "fixed_us": round(my - slope * mx, 2), "streaming_gbs": round(1e-3 / slope, 1)}
    del big
    log(f"[bench] plain read of {dec_bytes} B: median {pr_us:.1f} us, {read_peak:.0f} GB/s; "
        f"of 4 GiB: {pr4_us:.1f} us, {read_peak_4g:.0f} GB/s")

    # ---- the same step with randomized Walsh-Hadamard rotations --------------
    kqh = TA.Quantizer(Rkh, cfg.k_bits, cfg.k_variant, S, dev, "hadamard")
    vqh = TA.Quantizer(Rvh, cfg.v_bits, "mse", None, dev, "hadamard")
    for c in range(ncopy):
        TA.encode(kqh, kg, kcs[c])
        TA.encode(vqh, vg, vcs[c])
    had_ms, had_k = timed_steps(dec, (kqh, vqh), kcs, vcs, knew, vnew, q, out, args.warmup, args.steps)
    log(f"[bench] step with Hadamard rotations {had_ms:.4f} ms")
    del kcs, vcs
    torch.cuda.empty_cache()

    # ---- the other decode workloads -------------------------------------------
    # Each: fused decode steps back to back over rotating cache copies (enough
    # copies that the ones in rotation exceed the 256 MB last-level cache,
    # except for the 0.4 MB single-head cache, which is latency-bound), its
    # split launch alone after a 1 GiB read, and plain reads of as many bytes
    # under both conditions.
    configs = {}
    if not args.no_configs:
        for name, ncp, warm, steps in (("mse3_d128_4096_fp32", 1, 50, 200), ("llama8b_b4_32k", 12, 50, 200),
                                       ("llama8b_prod3_128k", 4, 50, 200), ("batch64_b2_16k", 3, 20, 50)):
            c = synth.WORKLOADS[name]
            kqc = TA.Quantizer(Rk, c.k_bits, c.k_variant, S if c.k_variant == "prod" else None, dev)
            vqc = TA.Quantizer(Rv, c.v_bits, "mse", None, dev)
            n_c = c.B * c.Hkv * c.T
            if n_c * c.d > (1 << 28):
                kx, vx = synth.make_kv_device(c, dev)      # too large to draw on the host quickly
            else:
                K_, V_ = synth.make_kv(c)
                tdt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
                kx = torch.from_numpy(K_.reshape(-1, d)).to(tdt).to(dev)
                vx = torch.from_numpy(V_.reshape(-1, d)).to(tdt).to(dev)
                del K_, V_
            kcc, vcc = packed_copies(kqc, vqc, kx, vx, n_c, ncp)
            qc = torch.from_numpy(synth.make_query(c)).to(dev)
            oc = torch.empty_like(qc)
            gn = np.random.default_rng(c.seed_base + 5)
            rows = c.B * c.Hkv
            tdt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
            kn_c = torch.from_numpy(synth.round_bf16(gn.standard_normal((rows, d)).astype(np.float32))).to(tdt).to(dev)
            vn_c = torch.from_numpy(synth.round_bf16(gn.standard_normal((rows, d)).astype(np.float32))).to(tdt).to(dev)
            dc = TA.Decoder(c.B, c.Hq, c.Hkv, c.T, dev)
            ms_c, k_c = timed_steps(dc, (kqc, vqc), kcc, vcc, kn_c, vn_c, qc, oc, warm, steps)
            kav = sum(k_c) / len(k_c)
            fl_c = flushed_split_us(dc, kqc, vqc, qc, kcc[0], vcc[0], oc, 5)
            by_c = n_c * bytes_per_token(c)
            rbufs = [torch.ones(by_c // 4, dtype=torch.float32, device=dev) for _ in range(ncp)]
            rd_b2b = read_back_to_back_us(rbufs, reps=30, warm=10)
            rd_fl = read_after_flush_us(rbufs[0])
            del rbufs, kcc, vcc, kx, vx
            torch.cuda.empty_cache()
            gbs = lambda us: round(by_c / (us * 1e-6) / 1e9, 1)
            frac = lambda us: round(by_c / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
            configs[name] = {
                "shape": f"B={c.B} Hkv={c.Hkv} Hq={c.Hq} T={c.T}", "keys": f"{c.k_variant}-{c.k_bits}",
                "values": f"mse-{c.v_bits}", "packed_cache_bytes": by_c, "cache_copies": ncp,
                "warmup": warm, "steps": steps,
                "step_us": round(ms_c * 1e3, 2), "step_gbs": gbs(ms_c * 1e3), "step_frac": frac(ms_c * 1e3),
                "split_us": round(kav, 2), "split_gbs": gbs(kav), "split_frac": frac(kav),
                "same_size_read_us": round(rd_b2b, 2), "split_over_read": round(rd_b2b / kav, 4),
                "split_after_flush_us": round(fl_c, 2), "split_after_flush_frac": frac(fl_c),
                "read_after_flush_us": round(rd_fl, 2),
            }
            log(f"[bench] {name}: {configs[name]}")

    # ---- inner-product search -------------------------------------------------
    # The first 2^20 key rows as a prod-4 database (index build = their
    # encode), 64 N(0,1) queries, top 10 each; recall 1@10 against the exact
    # top-1 of the unquantized rows.
    n_db, nq_s, k_s = 1 << 20, 64, 10
    db = TA.Packed(kq, n_db, dev)
    a_, b_ = Event(), Event()
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
    del ws_s, db
    torch.cuda.empty_cache()
    log(f"[bench] search: {search}")

    # ---- vectors longer than 128 coordinates: zero-padded chunks of 128 -------
    # d = 200 search (the pages' GloVe dimension; seeded N(0,1) vectors stand
    # in for the data set): 2^20 vectors, 64 queries, top 10, prod-4, recall
    # 1@10 against the exact top-1 of the unquantized vectors. d = 1536 index
    # build: 2^17 bf16 vectors encoded as 12 chunks each.
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed_base + 11)
    chunked = {}
    for dim, n_c, nq_c in ((200, 1 << 20, 64), (1536, 1 << 17, 64)):
        C = -(-dim // d)
        xr = torch.randn((n_c, dim), generator=gen, device=dev).to(torch.bfloat16)
        xp = torch.zeros((n_c, C * d), dtype=torch.bfloat16, device=dev)
        xp[:, :dim] = xr
        dbc = TA.Packed(kq, C * n_c, dev)
        TA.encode_chunked(kq, xp, C, dbc)
        a_.record()
        TA.encode_chunked(kq, xp, C, dbc)
        b_.record()
        torch.cuda.synchronize()
        bms = a_.elapsed_time(b_)
        qr = torch.randn((nq_c, dim), generator=gen, device=dev)
        qp = torch.zeros((nq_c, C * d), dtype=torch.float32, device=dev)
        qp[:, :dim] = qr
        ws_c = torch.empty(TA.L.tq_search_chunked_workspace(nq_c, n_c, k_s, C), dtype=torch.uint8, device=dev)
        for _ in range(3):
            TA.search_chunked(kq, qp, dbc, C, k_s, workspace=ws_c)
        reps = 10
        a_.record()
        for _ in range(reps):
            _, c_idx = TA.search_chunked(kq, qp, dbc, C, k_s, workspace=ws_c)
        b_.record()
        torch.cuda.synchronize()
        c_us = a_.elapsed_time(b_) / reps * 1e3
        top1 = (qr @ xr.float().T).argmax(dim=1)
        rec = float((c_idx == top1[:, None]).any(dim=1).float().mean())
        chunked[f"d{dim}"] = {
            "workload": f"{n_c} x d{dim} (bf16 N(0,1)) as {C} chunks of {d}, prod-{cfg.k_bits}; "
                        f"{nq_c} queries, top {k_s}",
            "index_build_ms": round(bms, 4), "build_mvec_s": round(n_c / (bms * 1e-3) / 1e6, 1),
            "search_us": round(c_us, 1), "gpairs_s": round(nq_c * n_c / (c_us * 1e-6) / 1e9, 1),
            "recall_1_at_10": round(rec, 4)}
        log(f"[bench] chunked d{dim}: {chunked[f'd{dim}']}")
        del xr, xp, dbc, ws_c
        torch.cuda.empty_cache()

    # ---- outlier-channel split workloads ("2.5-bit": 32 channels at 3 bits + 96
    # at 2, and "3.5-bit": 4 + 3; mse or prod keys, mse values, a norm (and
    # for prod a γ) per group) at the headline's shape: encode of the key
    # cache, the decode call (query operands, split attention, merge) over
    # three cache copies in turn, and the split-attention launch alone after
    # a 1 GiB read.
    split_res = {}
    if not args.no_split:
        for sname in ("gqa8_split25_128k_b4", "gqa8_split35_128k_b4", "gqa8_splitprod25_128k_b4",
                      "gqa8_splitprod35_128k_b4"):
            cs = synth.WORKLOADS[sname]
            sc = synth.split_constants(d)
            if cs.k_variant == "prod":
                kq6 = TA.Quantizer(None, cs.k_bits, "prod", None, dev,
                                   split=(sc["rk_o"], sc["rk_r"], sc["ch_k"], sc["sk_o"], sc["sk_r"]))
            else:
                kq6 = TA.Quantizer(None, cs.k_bits, "mse", None, dev, split=(sc["rk_o"], sc["rk_r"], sc["ch_k"]))
            vq6 = TA.Quantizer(None, cs.v_bits, "mse", None, dev, split=(sc["rv_o"], sc["rv_r"], sc["ch_v"]))
            K6, V6 = synth.make_kv(cs)
            k6 = torch.from_numpy(K6.reshape(-1, d)).to(torch.bfloat16).to(dev)
            v6 = torch.from_numpy(V6.reshape(-1, d)).to(torch.bfloat16).to(dev)
            del K6, V6
            n6 = cs.B * cs.Hkv * cs.T
            kc6, vc6 = packed_copies(kq6, vq6, k6, v6, n6, ncopy)
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
            us6 = flushed_split_us(dec6, kq6, vq6, q, kc6[0], vc6[0], out, 5)
            del kc6, vc6
            torch.cuda.empty_cache()
            tok6 = kq6.code_bytes + 8 + (16 + 8 if cs.k_variant == "prod" else 0) + vq6.code_bytes + 8
            by6 = n6 * tok6
            split_res[cs.name] = {
                "bytes_per_token_head": tok6, "packed_cache_bytes": by6,
                "decode_ms": round(ms6, 5), "decode_gbs": round(by6 / (ms6 * 1e-3) / 1e9, 1),
                "split_after_flush_us": round(us6, 2), "split_gbs": round(by6 / us6 / 1e3, 1),
                "frac": round(by6 / us6 / 1e3 / PEAK_HBM_GBS, 4),
                "encode_mvec_s": round(n6 / (enc6_ms * 1e-3) / 1e6, 1)}
            log(f"[bench] {cs.name}: {split_res[cs.name]}")
    del flush

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
                     "traffic": _traffic("attn_split_gqa8_prod4_128k.counters.json", "tq_decode.hip"),
                     "bytes_per_launch": dec_bytes, "avg_launch_us": round(k_avg, 2),
                     "launch_us_p10_p50_p90": [round(_pct(k_sorted, f), 2) for f in (0.1, 0.5, 0.9)],
                     "timed_in": "the headline's timed steps (events around each split launch)",
                     "after_read_flush_us": round(flushed_us, 2),
                     "frac_of_measured_read": round(achieved / read_peak, 4),
                     "cache_copies": ncopy},
        "steady_state": steady,
        "measured_read_peak": {"gbs": round(read_peak, 1), "bytes": dec_bytes, "us": round(pr_us, 2),
                               "gbs_4gib": round(read_peak_4g, 1),
                               "size_sweep": read_sweep,
                               "kernel": "tq_read_probe: plain coalesced read, 16-byte non-temporal loads",
                               "value_frac": round(value / read_peak, 4)},
        "configs": configs,
        "hadamard_step_ms": round(had_ms, 5),
        "hadamard_value": round(dec_bytes / (had_ms * 1e-3) / 1e9, 1),
        "search": search,
        "search_chunked": chunked,
        "outlier_split": split_res,
        "encode_mvec_s": enc,
        "encode_roofline": enc_roof,
        "encode_mfma": enc_mfma or None,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

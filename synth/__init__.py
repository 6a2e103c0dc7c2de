"""Seeded synthetic inputs shared by the HIP path and the oracle.

This module only draws random numbers and lays them out; it holds none of the
quantizer's arithmetic (no norms, no codebook, no quantization, no attention).
Every generator is `numpy.random.default_rng(seed)` (PCG64); data are drawn
as float32 standard normals (the constant matrices in float64) and rounded to
the stated storage dtype, so the GPU and the oracle consume the same bytes.

The random draws the method makes are inputs here, as the pages treat them:
  * the rotation is the orthogonal factor of a QR factorisation of an iid
    N(0,1) square matrix ("TurboQuant của Google…", omelet.tech, section
    "Trick đầu tiên: xoay ngẫu nhiên trước khi nén"); the sign of each column
    is fixed by the sign of R's diagonal so the draw is Haar-distributed;
  * the QJL projection is an iid N(0,1) square matrix ("内存厂商的噩梦来了…",
    wuyi.wiki, section 4.2; and the Gaussian-projection fact on "I Spent 31
    Hours On The Math Behind Turboquant…", onlylabs.fyi).

Workload shapes follow the Llama-3.1-8B cache shape the Baseten page uses
(8 KV heads, head dim 128; section "KV Cache: The problem").
"""
from __future__ import annotations

import dataclasses
import numpy as np

# Seeds for the per-layer constant matrices (one rotation for keys, one for
# values, one projection), and the per-config data seed base.
SEED_ROT_K = 1001
SEED_ROT_V = 1002
SEED_PROJ = 1003
SEED_HAD_K = 1004
SEED_HAD_V = 1005
# Outlier-channel split: per role (keys, values), the channel list and the
# rotations of the 32 outlier and the 96 regular channels.
SEED_SPLIT_CH_K = 1006
SEED_SPLIT_CH_V = 1007
SEED_SPLIT_ROT_K = (1008, 1009)
SEED_SPLIT_ROT_V = (1010, 1011)
SEED_SPLIT_PROJ_K = (1012, 1013)
SPLIT_OUTLIER_SCALE = 4.0


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round finite float64/float32 values to bfloat16 (round to nearest even).

    Returns the rounded values as float32 (exactly representable)."""
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    r = u >> 16
    r &= 1
    r += 0x7FFF
    u += r          # finite inputs cannot overflow 32 bits
    u &= 0xFFFF0000
    return u.view(np.float32)


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-exact."""
    return (np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def rotation(d: int, seed: int) -> np.ndarray:
    """Haar-random orthogonal d x d matrix as float32 (y = R @ u)."""
    g = rng(seed).standard_normal((d, d))
    q, r = np.linalg.qr(g)
    q = q * np.sign(np.diag(r))[None, :]
    return np.ascontiguousarray(q, dtype=np.float32)


def hadamard_rotation(d: int, seed: int) -> np.ndarray:
    """Randomized Walsh-Hadamard rotation H_d·diag(s)/√d as float32 (y = R @ u):
    H_d the Sylvester Hadamard matrix (d a power of two), s iid uniform ±1."""
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    if h.shape[0] != d:
        raise ValueError("d must be a power of two")
    s = rng(seed).choice(np.array([-1.0, 1.0]), size=d)
    return np.ascontiguousarray(h * s[None, :] / np.sqrt(d), dtype=np.float32)


def hadamard_constants(d: int = 128):
    """(Hadamard rotation for keys, for values, QJL projection), float32."""
    return hadamard_rotation(d, SEED_HAD_K), hadamard_rotation(d, SEED_HAD_V), projection(d, SEED_PROJ)


def projection(d: int, seed: int) -> np.ndarray:
    """iid N(0,1) d x d matrix as float32."""
    return np.ascontiguousarray(rng(seed).standard_normal((d, d)), dtype=np.float32)


def gaussian(shape, seed: int, dtype: str = "fp32") -> np.ndarray:
    """iid N(0,1) values rounded to `dtype` ("fp32" or "bf16"), returned as float32."""
    x = rng(seed).standard_normal(shape, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else x


def outlier_kv(B: int, H: int, T: int, d: int, seed: int, n_outliers: int = 4,
               scale: float = 10.0, dtype: str = "bf16") -> np.ndarray:
    """[B,H,T,d] N(0,1) cache with `n_outliers` seeded channels per head scaled.

    The same channels are scaled for every token of a head (a per-channel
    outlier pattern); channels are drawn without replacement per head."""
    g = rng(seed)
    x = g.standard_normal((B, H, T, d), dtype=np.float32)
    for h in range(H):
        ch = g.choice(d, size=n_outliers, replace=False)
        x[:, h, :, ch] *= np.float32(scale)
    return round_bf16(x) if dtype == "bf16" else x


def lognormal_kv(B: int, H: int, T: int, d: int, seed: int, sigma: float = 0.5,
                 dtype: str = "bf16") -> np.ndarray:
    """[B,H,T,d] N(0,I) directions times per-(b,h,t) LogNormal(0, sigma) scales."""
    g = rng(seed)
    x = g.standard_normal((B, H, T, d), dtype=np.float32)
    s = g.lognormal(0.0, sigma, size=(B, H, T, 1)).astype(np.float32)
    x *= s
    return round_bf16(x) if dtype == "bf16" else x


def outlier_channels(d: int, seed: int, n: int = 32) -> np.ndarray:
    """`n` distinct channels out of d, drawn without replacement, in draw order."""
    return rng(seed).choice(d, size=n, replace=False).astype(np.int64)


def split_constants(d: int = 128):
    """Per role, the outlier-channel split's inputs: dict(ch_k, rk_o, rk_r,
    ch_v, rv_o, rv_r, sk_o, sk_r) with ch_* 32 channel indices, r*_o (32x32)
    and r*_r (96x96) rotations drawn as the dense one is, and the keys' QJL
    projections sk_o (32x32) and sk_r (96x96) for prod keys."""
    n = 32
    return dict(ch_k=outlier_channels(d, SEED_SPLIT_CH_K, n), rk_o=rotation(n, SEED_SPLIT_ROT_K[0]),
                rk_r=rotation(d - n, SEED_SPLIT_ROT_K[1]), ch_v=outlier_channels(d, SEED_SPLIT_CH_V, n),
                rv_o=rotation(n, SEED_SPLIT_ROT_V[0]), rv_r=rotation(d - n, SEED_SPLIT_ROT_V[1]),
                sk_o=projection(n, SEED_SPLIT_PROJ_K[0]), sk_r=projection(d - n, SEED_SPLIT_PROJ_K[1]))


def split_kv(B: int, H: int, T: int, d: int, seed: int, channels, scale: float = SPLIT_OUTLIER_SCALE,
             dtype: str = "bf16") -> np.ndarray:
    """[B,H,T,d] N(0,1) cache whose listed channels (the same in every head)
    are scaled by `scale`: the per-channel outlier pattern the split is for."""
    x = rng(seed).standard_normal((B, H, T, d), dtype=np.float32)
    x[..., np.asarray(channels)] *= np.float32(scale)
    return round_bf16(x) if dtype == "bf16" else x


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    """One decode workload: the cache shape, the quantizers and the data recipe."""
    name: str
    B: int
    Hkv: int
    Hq: int
    T: int
    d: int
    k_variant: str      # "mse" or "prod"
    k_bits: int         # total bits per coordinate for keys
    v_bits: int         # bits per coordinate for values (MSE)
    recipe: str         # "gaussian", "outlier", "lognormal", "split"
    dtype: str          # storage dtype of the raw K/V ("fp32" or "bf16")
    seed_base: int
    split: bool = False  # outlier-channel split: k_bits / v_bits are the regular channels' bits

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


# The workloads, by name. "K" is 1024 tokens.
_ALL = (
    DecodeConfig("mse3_d128_4096_fp32", 1, 1, 1, 4096, 128, "mse", 3, 3, "gaussian", "fp32", 10),
    DecodeConfig("llama8b_b4_32k", 1, 8, 32, 32768, 128, "mse", 4, 4, "outlier", "bf16", 20),
    DecodeConfig("llama8b_prod3_128k", 1, 8, 32, 131072, 128, "prod", 3, 3, "outlier", "bf16", 30),
    DecodeConfig("batch64_b2_16k", 64, 8, 32, 16384, 128, "mse", 2, 2, "lognormal", "bf16", 40),
    DecodeConfig("gqa8_prod4_128k_b4", 4, 8, 64, 131072, 128, "prod", 4, 4, "gaussian", "bf16", 50),
    # outlier-channel split ("2.5-bit": 32 channels at 3 bits + 96 at 2;
    # "3.5-bit": 4 + 3), mse keys and values, the benchmark's shape
    DecodeConfig("gqa8_split25_128k_b4", 4, 8, 64, 131072, 128, "mse", 2, 2, "split", "bf16", 60, True),
    DecodeConfig("gqa8_split35_128k_b4", 4, 8, 64, 131072, 128, "mse", 3, 3, "split", "bf16", 70, True),
    # the same split with prod keys (each group a prod instance: 32 channels
    # at 3 bits + 96 at 2, or 4 + 3, counting the sketch bit), mse values
    DecodeConfig("gqa8_splitprod25_128k_b4", 4, 8, 64, 131072, 128, "prod", 2, 2, "split", "bf16", 80, True),
    DecodeConfig("gqa8_splitprod35_128k_b4", 4, 8, 64, 131072, 128, "prod", 3, 3, "split", "bf16", 90, True),
)
WORKLOADS = {c.name: c for c in _ALL}
# The five unsplit decode workloads, smallest first.
DECODE_WORKLOADS = [c.name for c in _ALL if not c.split]


def make_kv(cfg: DecodeConfig, T: int | None = None, B: int | None = None):
    """Raw K and V caches [B,Hkv,T,d] (float32 values, bf16-exact when dtype is bf16).

    `T`/`B` override the config's context length / batch for smaller cases
    that keep the same value distribution."""
    T = cfg.T if T is None else T
    B = cfg.B if B is None else B
    sk, sv = cfg.seed_base + 0, cfg.seed_base + 1
    if cfg.recipe == "gaussian":
        k = gaussian((B, cfg.Hkv, T, cfg.d), sk, cfg.dtype)
        v = gaussian((B, cfg.Hkv, T, cfg.d), sv, cfg.dtype)
    elif cfg.recipe == "outlier":
        k = outlier_kv(B, cfg.Hkv, T, cfg.d, sk, dtype=cfg.dtype)
        v = outlier_kv(B, cfg.Hkv, T, cfg.d, sv, dtype=cfg.dtype)
    elif cfg.recipe == "lognormal":
        k = lognormal_kv(B, cfg.Hkv, T, cfg.d, sk, dtype=cfg.dtype)
        v = lognormal_kv(B, cfg.Hkv, T, cfg.d, sv, dtype=cfg.dtype)
    elif cfg.recipe == "split":
        c = split_constants(cfg.d)
        k = split_kv(B, cfg.Hkv, T, cfg.d, sk, c["ch_k"], dtype=cfg.dtype)
        v = split_kv(B, cfg.Hkv, T, cfg.d, sv, c["ch_v"], dtype=cfg.dtype)
    else:
        raise ValueError(cfg.recipe)
    return k, v


def make_query(cfg: DecodeConfig, B: int | None = None) -> np.ndarray:
    """fp32 N(0,1) queries [B,Hq,d]."""
    B = cfg.B if B is None else B
    return gaussian((B, cfg.Hq, cfg.d), cfg.seed_base + 2, "fp32")


def constants(d: int = 128):
    """(rotation for keys, rotation for values, QJL projection), float32."""
    return rotation(d, SEED_ROT_K), rotation(d, SEED_ROT_V), projection(d, SEED_PROJ)


def make_kv_device(cfg: DecodeConfig, device, T: int | None = None, B: int | None = None):
    """Raw K and V caches [B*Hkv*T, d] drawn on the device by a seeded torch
    generator with the same recipe as make_kv (N(0,1); the outlier recipe's
    4 channels per head ×10; the log-normal recipe's per-token LogNormal(0,
    0.5) scales), stored as cfg.dtype (bfloat16 by round-to-nearest-even, or
    float32). The numbers differ from make_kv's (another generator); they
    serve timing runs of caches too large to draw on the host quickly, never
    a comparison with the oracle."""
    import torch

    T = cfg.T if T is None else T
    B = cfg.B if B is None else B
    out = []
    for role in (0, 1):
        g = torch.Generator(device=device).manual_seed(cfg.seed_base + role)
        x = torch.randn((B, cfg.Hkv, T, cfg.d), generator=g, device=device, dtype=torch.float32)
        if cfg.recipe == "outlier":
            for h in range(cfg.Hkv):
                ch = torch.randperm(cfg.d, generator=g, device=device)[:4]
                x[:, h, :, ch] *= 10.0
        elif cfg.recipe == "lognormal":
            s = torch.randn((B, cfg.Hkv, T, 1), generator=g, device=device, dtype=torch.float32)
            x *= torch.exp(0.5 * s)
        elif cfg.recipe != "gaussian":
            raise ValueError(cfg.recipe)
        x = x.reshape(-1, cfg.d)
        out.append(x.to(torch.bfloat16) if cfg.dtype == "bf16" else x)
    return out[0], out[1]

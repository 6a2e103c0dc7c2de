"""TurboQuant oracle: a plain, slow, float64 statement of what the method computes.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module. It shares no code with the HIP path
(the library under kv_cache_vector_06_amd/ and include/), and the HIP path
never imports it.

Pages cited below, by key:
  [DG]  "The Distortion Guarantee — How Good Is This?"
        (igniting.github.io/turboquant/slides/section-09)
  [B31] "I Spent 31 Hours On The Math Behind Turboquant So You Dont Have To"
        (onlylabs.fyi, Baseten research)
  [OM]  "TurboQuant của Google: nén KV cache 6 lần, hay một paper cũ 9 tháng
        được PR lại?" (omelet.tech)
  [WY]  "内存厂商的噩梦来了：谷歌一篇论文如何让 KV Cache 内存占用缩小六倍"
        (wuyi.wiki)

Every function is float64. Library primitives used as single steps:
`scipy.special.betainc` (the regularized incomplete beta function, i.e. the
CDF of a Beta law), `numpy` matrix products, `argmin`, `packbits`.

Readings of points the pages leave open (each is listed in the design doc too):
  * codebook density: the exact law of one coordinate of a uniform unit
    vector in R^d, f_d(x) = C_d (1-x^2)^((d-3)/2) on [-1,1] ([OM] section
    "Trick đầu tiên…", eq. f(x)); C_d is the normaliser Γ(d/2)/(√π Γ((d-1)/2)).
  * ties in nearest-centroid search go to the lower index.
  * a zero vector has norm 0 and unit direction u = 0; every later step then
    follows its plain definition.
  * prod keeps the 1-bit QJL sketch of the residual in the original space,
    r = u - Πᵀ c[idx], with projection S (d x d), bit_j = [ (S r)_j >= 0 ].
  * the prod reconstruction scale is √(π/2)/d · ‖r‖ (derived in
    `dequant_prod`; the pages print the estimator without it).
  * bits per coordinate: mse uses b bits; prod uses b-1 bits of Lloyd-Max
    plus the 1-bit sketch ([OM] section on QJL; [WY] section 4.3).
  * packing: code j of a vector occupies bits [j·b, j·b+b) of that vector's
    byte string, least significant bit first; sketch bit j is bit j.
  * outlier-channel split ([OM] section on the 3.5-bit experiment): two
    independent TurboQuant-mse instances, one on the 32 outlier channels at
    b+1 bits (codebook for d = 32) and one on the other 96 at b bits
    (codebook for d = 96), each with its own norm and rotation. The channel
    list is the caller's (the pages give no selection rule). The printed
    average, (32·3 + 96·2)/128 = 2.5, is 2.25 bits of codes; the other 0.25
    bit per channel matches two 16-bit group norms. The counts and widths
    are kept as printed.
  * outlier-channel split with prod keys: the same two groups, each a
    TurboQuant-prod instance at its group's width — the outlier group at
    bits+1 (bits of Lloyd-Max, d = 32 codebook, plus a 1-bit sketch with its
    own 32×32 Gaussian S_o) and the regular group at bits (bits-1 of
    Lloyd-Max, d = 96, plus a 1-bit sketch with a 96×96 S_r); each group keeps
    its own norm and γ. The sketch bits sit at the groups' positions of the
    split layout, and the correction scale √(π/2)/d_g uses the group's d_g.
  * vectors longer than 128 coordinates ([WY] section 6.4 searches d = 200
    and d = 1536): zero-padded to C = ceil(d/128)·128 coordinates and cut into
    C chunks of 128, each quantized on its own by the same 128-coordinate
    quantizer (own norm; own sketch and γ for prod). The estimate of ⟨q, x⟩ is
    Σ_c ⟨q_c, x̃_c⟩, i.e. the inner product with the chunks' dequantized
    vectors laid side by side.
"""
from __future__ import annotations

import math
import numpy as np
from scipy.special import betainc

__all__ = [
    "coord_norm_const", "coord_density", "coord_mass", "coord_first_moment",
    "coord_second_moment", "lloyd_max", "codebook_mse", "nearest_centroid",
    "pack_codes", "unpack_codes", "pack_signs", "unpack_signs",
    "encode_mse", "encode_prod", "dequant_mse", "dequant_prod",
    "attention", "decode_attention", "fwht", "hadamard_rotate",
    "search_topk", "recall_1_at_k", "chunk_vectors", "unchunk_vectors",
    "SPLIT_OUTLIERS", "split_positions", "split_widths", "pack_split", "unpack_split",
    "encode_split", "dequant_split", "encode_split_prod", "dequant_split_prod", "pack_positions",
]


# ---------------------------------------------------------------------------
# The coordinate law after a random rotation  ([OM] "Trick đầu tiên…", eq. f(x))
# ---------------------------------------------------------------------------

def coord_norm_const(d: int) -> float:
    """C_d such that C_d (1-x^2)^((d-3)/2) integrates to 1 on [-1, 1]."""
    return math.exp(math.lgamma(d / 2) - math.lgamma((d - 1) / 2)) / math.sqrt(math.pi)


def coord_density(x, d: int):
    """f_d(x) = C_d (1-x^2)^((d-3)/2): one coordinate of a uniform unit vector."""
    x = np.asarray(x, dtype=np.float64)
    return coord_norm_const(d) * np.clip(1.0 - x * x, 0.0, None) ** ((d - 3) / 2)


def _cdf(x, d: int):
    # (1+X)/2 ~ Beta((d-1)/2, (d-1)/2) when X has density f_d.
    a = (d - 1) / 2
    return betainc(a, a, (1.0 + np.clip(np.asarray(x, np.float64), -1.0, 1.0)) / 2)


def coord_mass(a, b, d: int):
    """∫_a^b f_d(x) dx."""
    return _cdf(b, d) - _cdf(a, d)


def coord_first_moment(a, b, d: int):
    """∫_a^b x f_d(x) dx = C_d/(d-1) [(1-a²)^((d-1)/2) - (1-b²)^((d-1)/2)]."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    e = (d - 1) / 2
    g = lambda x: np.clip(1.0 - x * x, 0.0, None) ** e
    return coord_norm_const(d) / (d - 1) * (g(a) - g(b))


def coord_second_moment(a, b, d: int):
    """∫_a^b x² f_d(x) dx.

    Uses (1-x²) f_d = ((d-1)/d) f_{d+2}, so ∫x² f_d = ∫f_d - ((d-1)/d) ∫f_{d+2}."""
    return coord_mass(a, b, d) - (d - 1) / d * coord_mass(a, b, d + 2)


# ---------------------------------------------------------------------------
# Lloyd-Max codebook  ([OM] "Lloyd-Max quantizer: chia bucket đúng chỗ", eq. C(f,b))
# ---------------------------------------------------------------------------

def lloyd_max(d: int, bits: int, tol: float = 1e-13, max_iter: int = 200000, init=None):
    """Lloyd-Max quantizer of f_d with 2^bits levels.

    Minimises Σ_i ∫_{cell i} (x - c_i)² f_d(x) dx by the two Lloyd conditions:
    cell edges at midpoints of neighbouring centroids, centroids at the
    conditional mean of their cell. Starts from the Gaussian N(0,1/d)
    quantiles at (i+1/2)/K unless `init` is given.

    Returns (centroids[K] ascending, boundaries[K-1], D) where D = d × the
    per-coordinate MSE, i.e. the expected ‖u - ũ‖² of a unit vector.
    bits = 0 gives the single centroid 0 and D = 1. Iteration stops when no
    centroid moves by more than `tol` × (1/√d), the coordinate's scale.
    """
    if bits == 0:
        return np.zeros(1), np.zeros(0), 1.0
    K = 1 << bits
    if init is None:
        from scipy.stats import norm
        c = norm.ppf((np.arange(K) + 0.5) / K) / math.sqrt(d)
    else:
        c = np.array(init, dtype=np.float64)
    for _ in range(max_iter):
        t = 0.5 * (c[:-1] + c[1:])
        lo = np.concatenate(([-1.0], t))
        hi = np.concatenate((t, [1.0]))
        c_new = coord_first_moment(lo, hi, d) / coord_mass(lo, hi, d)
        delta = np.max(np.abs(c_new - c))
        c = c_new
        if delta < tol / math.sqrt(d):
            break
    else:
        raise RuntimeError("Lloyd-Max did not converge")
    # f_d is even, so the optimum is antisymmetric; make it exactly so, which
    # puts the middle boundary at 0 and lets a tie at y = 0 resolve to the
    # lower index as nearest_centroid states.
    c = 0.5 * (c - c[::-1])
    t = 0.5 * (c[:-1] + c[1:])
    return c, t, codebook_mse(c, t, d)


def codebook_mse(c, t, d: int) -> float:
    """d × Σ_i ∫_{t_{i-1}}^{t_i} (x - c_i)² f_d(x) dx  (MSE of a unit vector)."""
    c = np.asarray(c, np.float64)
    lo = np.concatenate(([-1.0], t))
    hi = np.concatenate((t, [1.0]))
    per = (coord_second_moment(lo, hi, d) - 2 * c * coord_first_moment(lo, hi, d)
           + c * c * coord_mass(lo, hi, d))
    return float(d * np.sum(per))


def nearest_centroid(y, c):
    """idx = argmin_i |y - c_i|, ties to the lower index ([OM] Lloyd-Max section)."""
    y = np.asarray(y, np.float64)
    return np.argmin(np.abs(y[..., None] - np.asarray(c, np.float64)), axis=-1).astype(np.int64)


# ---------------------------------------------------------------------------
# Bit packing: LSB-first stream per vector
# ---------------------------------------------------------------------------

def pack_codes(idx, bits: int) -> np.ndarray:
    """[N, d] codes → [N, d·bits/8] bytes; code j at bits [j·bits, j·bits+bits)."""
    idx = np.asarray(idx, np.int64)
    N, d = idx.shape
    if bits == 0:
        return np.zeros((N, 0), np.uint8)
    planes = (idx[:, :, None] >> np.arange(bits)) & 1          # [N, d, bits]
    return np.packbits(planes.reshape(N, d * bits).astype(np.uint8), axis=1, bitorder="little")


def unpack_codes(packed, d: int, bits: int) -> np.ndarray:
    packed = np.asarray(packed, np.uint8)
    N = packed.shape[0]
    if bits == 0:
        return np.zeros((N, d), np.int64)
    stream = np.unpackbits(packed, axis=1, bitorder="little")[:, : d * bits]
    planes = stream.reshape(N, d, bits).astype(np.int64)
    return np.sum(planes << np.arange(bits), axis=-1)


def pack_signs(z) -> np.ndarray:
    """[N, m] real → [N, m/8] bytes, bit j = 1 iff z_j >= 0 (sign(0) = +1)."""
    return np.packbits((np.asarray(z) >= 0).astype(np.uint8), axis=1, bitorder="little")


def unpack_signs(packed, m: int) -> np.ndarray:
    """→ [N, m] of ±1.0."""
    bits = np.unpackbits(np.asarray(packed, np.uint8), axis=1, bitorder="little")[:, :m]
    return np.where(bits == 1, 1.0, -1.0)


# ---------------------------------------------------------------------------
# Randomized Walsh-Hadamard rotation  ([WY] section 4.3: the WHT as the
# efficient replacement of the dense rotation matrix)
# ---------------------------------------------------------------------------

def fwht(v):
    """Unnormalised Walsh-Hadamard transform along the last axis: v ↦ H v with
    H the Sylvester Hadamard matrix (H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]],
    so H[i][j] = (-1)^popcount(i & j)); the length must be a power of two.
    Butterflies of span 1, 2, 4, ...: pairs (a, b) at distance h become
    (a + b, a - b)."""
    v = np.array(v, dtype=np.float64, copy=True)
    n = v.shape[-1]
    if n & (n - 1):
        raise ValueError("length must be a power of two")
    lead = v.shape[:-1]
    h = 1
    while h < n:
        w = v.reshape(lead + (n // (2 * h), 2, h))
        a = w[..., 0, :].copy()
        b = w[..., 1, :].copy()
        w[..., 0, :] = a + b
        w[..., 1, :] = a - b
        v = w.reshape(lead + (n,))
        h *= 2
    return v


def hadamard_rotate(u, signs):
    """y = H diag(s) u / √d, the randomized Hadamard rotation of the rows of u
    (s the ±1 sign vector). It is orthogonal since H Hᵀ = d I."""
    u = np.asarray(u, np.float64)
    s = np.asarray(signs, np.float64)
    return fwht(u * s) / math.sqrt(u.shape[-1])


# ---------------------------------------------------------------------------
# Encode / dequantize
# ---------------------------------------------------------------------------

def _unit(X):
    X = np.asarray(X, np.float64)
    n = np.sqrt(np.sum(X * X, axis=1))
    u = np.zeros_like(X)
    nz = n > 0
    u[nz] = X[nz] / n[nz, None]
    return n, u


def encode_mse(X, rot, c, bits: int):
    """TurboQuant-mse encode ([DG] "rotate, quantize"; [OM] rotation and Lloyd-Max sections).

    n = ‖x‖ is kept unquantized (the HN thread on qwik-news notes the norm is
    one scalar per vector); u = x/n; y = Π u; idx_j = nearest centroid of y_j.
    Returns dict(codes=[N, d·bits/8] uint8, norms=[N] float64, idx=[N,d], y=[N,d]).
    """
    n, u = _unit(X)
    y = u @ np.asarray(rot, np.float64).T
    idx = nearest_centroid(y, c)
    return dict(codes=pack_codes(idx, bits), norms=n, idx=idx, y=y)


def encode_prod(X, rot, proj, c_m, bits: int):
    """TurboQuant-prod encode ([OM] QJL section; [WY] sections 4.2-4.3).

    (bits-1)-bit mse quantizer on u, residual r = u - Πᵀ c[idx] in the
    original space, γ = ‖r‖, and the 1-bit sketch sign(S r).
    `c_m` is the (bits-1)-bit codebook (the single centroid 0 when bits == 1).
    """
    bm = bits - 1
    n, u = _unit(X)
    R = np.asarray(rot, np.float64)
    S = np.asarray(proj, np.float64)
    y = u @ R.T
    idx = nearest_centroid(y, c_m)
    u_mse = np.asarray(c_m, np.float64)[idx] @ R           # Πᵀ c[idx], row form
    r = u - u_mse
    gamma = np.sqrt(np.sum(r * r, axis=1))
    z = r @ S.T
    return dict(codes=pack_codes(idx, bm), norms=n, qjl=pack_signs(z), gammas=gamma,
                idx=idx, y=y, z=z)


def dequant_mse(codes, norms, rot, c, bits: int):
    """x̃ = n Πᵀ c[idx]."""
    d = np.asarray(rot).shape[0]
    idx = unpack_codes(codes, d, bits)
    return np.asarray(norms, np.float64)[:, None] * (np.asarray(c, np.float64)[idx] @ np.asarray(rot, np.float64))


def dequant_prod(codes, norms, qjl, gammas, rot, proj, c_m, bits: int):
    """x̃ = n (Πᵀ c[idx] + √(π/2)/d · γ · Sᵀ s), s_j = ±1.

    Scale derivation (the pages print the correction term without it): for
    one Gaussian row σ of S, (⟨σ,y⟩, ⟨σ,r⟩) is jointly Gaussian with
    covariance from the Baseten page's fact S·x ~ N(0, ‖x‖² I), so
    E[⟨σ,y⟩ sign⟨σ,r⟩] = √(2/π) ⟨y,r⟩/‖r‖. Summing d rows and multiplying by
    √(π/2) ‖r‖ / d makes E⟨y, x̃⟩ = ⟨y, x⟩, the unbiasedness [OM] states in
    its QJL section.
    """
    d = np.asarray(rot).shape[0]
    m = np.asarray(proj).shape[0]
    bm = bits - 1
    idx = unpack_codes(codes, d, bm)
    s = unpack_signs(qjl, m)
    base = np.asarray(c_m, np.float64)[idx] @ np.asarray(rot, np.float64)
    corr = (math.sqrt(math.pi / 2) / m) * np.asarray(gammas, np.float64)[:, None] * (s @ np.asarray(proj, np.float64))
    return np.asarray(norms, np.float64)[:, None] * (base + corr)


# ---------------------------------------------------------------------------
# Outlier-channel split  ([OM] section "Thực nghiệm: 3.5 bit…": the 128
# channels of a head form two groups, 32 outlier channels at one bit more than
# the 96 regular ones; e.g. 32 at 3 bits + 96 at 2 bits)
# ---------------------------------------------------------------------------

SPLIT_OUTLIERS = 32


def split_positions(d: int = 128):
    """Where each group's coordinates sit in a split vector's code string (a
    storage layout, ours): position p holds an outlier coordinate iff
    p mod 8 < 2. Returns (P_o, P_r): outlier coordinate k sits at P_o[k],
    regular coordinate k at P_r[k], each group in its own order."""
    p = np.arange(d)
    return p[p % 8 < 2], p[p % 8 >= 2]


def split_widths(bits: int, d: int = 128):
    """Code width of each position: bits + 1 at outlier positions, bits elsewhere."""
    w = np.full(d, bits, np.int64)
    w[split_positions(d)[0]] = bits + 1
    return w


def pack_split(idx, bits: int) -> np.ndarray:
    """[N, d] codes in position order → [N, (d·bits + 32)/8] bytes: the codes
    one after another, position 0 first, each least significant bit first,
    with the width of its position."""
    idx = np.asarray(idx, np.int64)
    N, d = idx.shape
    w = split_widths(bits, d)
    stream = []
    for p in range(d):
        for k in range(w[p]):
            stream.append((idx[:, p] >> k) & 1)
    return np.packbits(np.stack(stream, axis=1).astype(np.uint8), axis=1, bitorder="little")


def unpack_split(packed, bits: int, d: int = 128) -> np.ndarray:
    packed = np.asarray(packed, np.uint8)
    w = split_widths(bits, d)
    stream = np.unpackbits(packed, axis=1, bitorder="little").astype(np.int64)
    out = np.zeros((packed.shape[0], d), np.int64)
    at = 0
    for p in range(d):
        for k in range(w[p]):
            out[:, p] |= stream[:, at] << k
            at += 1
    return out


def _regular_channels(ch_o, d: int):
    mask = np.ones(d, bool)
    mask[np.asarray(ch_o)] = False
    return np.nonzero(mask)[0]


def encode_split(X, ch_o, rot_o, rot_r, c_o, c_r, bits: int):
    """Outlier-channel split encode: two independent TurboQuant-mse instances.
    The outlier channels ch_o (32 raw channel indices, in the order that
    rot_o's columns follow) are encoded with their own norm, rotation rot_o
    (32×32) and Lloyd-Max codebook c_o (d = 32, bits + 1 bits); the other 96
    channels, in increasing order, with rot_r (96×96) and c_r (d = 96, bits).
    Returns dict(codes=[N, (128·bits+32)/8] uint8, norms=[N, 2] (outlier,
    regular), idx=[N,128] in position order, idx_o, idx_r, and each group's
    rotated unit coordinates y_o, y_r)."""
    X = np.asarray(X, np.float64)
    d = X.shape[1]
    ch_r = _regular_channels(ch_o, d)
    eo = encode_mse(X[:, np.asarray(ch_o)], rot_o, c_o, bits + 1)
    er = encode_mse(X[:, ch_r], rot_r, c_r, bits)
    P_o, P_r = split_positions(d)
    idx = np.zeros((X.shape[0], d), np.int64)
    idx[:, P_o] = eo["idx"]
    idx[:, P_r] = er["idx"]
    return dict(codes=pack_split(idx, bits), norms=np.stack([eo["norms"], er["norms"]], axis=1), idx=idx,
                idx_o=eo["idx"], idx_r=er["idx"], y_o=eo["y"], y_r=er["y"])


def dequant_split(codes, norms, ch_o, rot_o, rot_r, c_o, c_r, bits: int, d: int = 128):
    """x̃ with x̃[ch_o] = n_o Π_oᵀ c_o[idx_o] and x̃[ch_r] = n_r Π_rᵀ c_r[idx_r]."""
    idx = unpack_split(codes, bits, d)
    P_o, P_r = split_positions(d)
    norms = np.asarray(norms, np.float64)
    ch_r = _regular_channels(ch_o, d)
    out = np.zeros((idx.shape[0], d))
    out[:, np.asarray(ch_o)] = norms[:, :1] * (np.asarray(c_o, np.float64)[idx[:, P_o]] @ np.asarray(rot_o, np.float64))
    out[:, ch_r] = norms[:, 1:] * (np.asarray(c_r, np.float64)[idx[:, P_r]] @ np.asarray(rot_r, np.float64))
    return out


def pack_positions(z_o, z_r, d: int = 128) -> np.ndarray:
    """The two groups' sketch values laid out by position (outlier coordinate
    k at P_o[k], regular k at P_r[k]) and packed as sign bits, bit p = 1 iff
    the value at position p is >= 0."""
    P_o, P_r = split_positions(d)
    z = np.zeros((np.asarray(z_o).shape[0], d))
    z[:, P_o] = z_o
    z[:, P_r] = z_r
    return pack_signs(z)


def encode_split_prod(X, ch_o, rot_o, rot_r, proj_o, proj_r, c_o, c_r, bits: int):
    """Outlier-channel split with prod keys: two independent TurboQuant-prod
    instances. The outlier channels ch_o (in the order of rot_o's columns) at
    bits + 1 (Lloyd-Max codebook c_o for d = 32 at `bits` bits, sketch S_o =
    proj_o, 32×32), the other 96 channels in increasing order at `bits`
    (c_r for d = 96 at bits - 1 bits, S_r = proj_r, 96×96). The Lloyd-Max
    codes form the split code string of width bits - 1 (outlier positions
    `bits` wide); the sketch bits sit at the same positions.
    Returns dict(codes, norms=[N,2], qjl=[N,16], gammas=[N,2] (outlier,
    regular), idx (position order), y_o, y_r, z_o, z_r)."""
    X = np.asarray(X, np.float64)
    d = X.shape[1]
    ch_r = _regular_channels(ch_o, d)
    eo = encode_prod(X[:, np.asarray(ch_o)], rot_o, proj_o, c_o, bits + 1)
    er = encode_prod(X[:, ch_r], rot_r, proj_r, c_r, bits)
    P_o, P_r = split_positions(d)
    idx = np.zeros((X.shape[0], d), np.int64)
    idx[:, P_o] = eo["idx"]
    idx[:, P_r] = er["idx"]
    return dict(codes=pack_split(idx, bits - 1), norms=np.stack([eo["norms"], er["norms"]], axis=1),
                qjl=pack_positions(eo["z"], er["z"], d), gammas=np.stack([eo["gammas"], er["gammas"]], axis=1),
                idx=idx, y_o=eo["y"], y_r=er["y"], z_o=eo["z"], z_r=er["z"])


def dequant_split_prod(codes, norms, qjl, gammas, ch_o, rot_o, rot_r, proj_o, proj_r, c_o, c_r, bits: int,
                       d: int = 128):
    """x̃[ch_o] = n_o (Π_oᵀ c_o[idx_o] + √(π/2)/32 · γ_o S_oᵀ s_o) and
    x̃[ch_r] = n_r (Π_rᵀ c_r[idx_r] + √(π/2)/96 · γ_r S_rᵀ s_r), s_g the
    group's sketch signs read at its positions."""
    idx = unpack_split(codes, bits - 1, d)
    P_o, P_r = split_positions(d)
    s = unpack_signs(qjl, d)
    norms = np.asarray(norms, np.float64)
    gammas = np.asarray(gammas, np.float64)
    ch_r = _regular_channels(ch_o, d)
    out = np.zeros((idx.shape[0], d))
    for ch, P, R, S, c, col in ((np.asarray(ch_o), P_o, rot_o, proj_o, c_o, 0), (ch_r, P_r, rot_r, proj_r, c_r, 1)):
        R = np.asarray(R, np.float64)
        S = np.asarray(S, np.float64)
        base = np.asarray(c, np.float64)[idx[:, P]] @ R
        corr = (math.sqrt(math.pi / 2) / S.shape[0]) * gammas[:, col:col + 1] * (s[:, P] @ S)
        out[:, ch] = norms[:, col:col + 1] * (base + corr)
    return out


# ---------------------------------------------------------------------------
# Attention  ([B31] "KV Cache: The problem": softmax(Q·Kᵀ/√d)·V)
# ---------------------------------------------------------------------------

def attention(q, K, V, scale: float):
    """One query over T keys/values: softmax(K q · scale) V, float64."""
    q = np.asarray(q, np.float64)
    s = np.asarray(K, np.float64) @ q * scale
    p = np.exp(s - np.max(s))
    p /= np.sum(p)
    return p @ np.asarray(V, np.float64)


def decode_attention(q, K, V, scale: float, ctx_lens=None, heads=None):
    """q [B,Hq,d]; K,V [B,Hkv,T,d] (already dequantized); query head h reads
    KV head h // (Hq/Hkv). `ctx_lens[b]` limits the tokens of batch b.
    `heads` optionally restricts the evaluation to a list of (b, h) pairs.
    Returns out [B,Hq,d] (rows not evaluated are NaN)."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.full((B, Hq, d), np.nan)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in pairs:
        L = K.shape[2] if ctx_lens is None else int(ctx_lens[b])
        out[b, h] = attention(q[b, h], K[b, h // G, :L], V[b, h // G, :L], scale)
    return out


# ---------------------------------------------------------------------------
# Inner-product vector search over a packed database  ([WY] section 6.4:
# TurboQuant used for nearest-neighbour search by inner product, scored by
# recall 1@k)
# ---------------------------------------------------------------------------

def search_topk(Q, X, k: int):
    """For each query row q of Q, the k rows x of X with the largest ⟨q, x⟩,
    best first; equal scores are ordered by the lower row index. X is the
    database as the searcher sees it (for a packed database, its dequantized
    vectors). Returns (scores [nq, k] float64, index [nq, k] int64)."""
    Q = np.asarray(Q, np.float64)
    X = np.asarray(X, np.float64)
    S = Q @ X.T
    n = X.shape[0]
    idx = np.empty((Q.shape[0], k), np.int64)
    for i in range(Q.shape[0]):
        # sort by (-score, index): lexsort takes the last key as the primary one
        order = np.lexsort((np.arange(n), -S[i]))
        idx[i] = order[:k]
    return np.take_along_axis(S, idx, axis=1), idx


def recall_1_at_k(true_top1, found):
    """Fraction of queries whose true nearest neighbour (true_top1[i]) is among
    the k indices found[i] (recall 1@k)."""
    true_top1 = np.asarray(true_top1).reshape(-1)
    found = np.asarray(found)
    return float(np.mean([true_top1[i] in found[i] for i in range(found.shape[0])]))


# ---------------------------------------------------------------------------
# Vectors longer than one 128-coordinate block  ([WY] section 6.4: search over
# 200-dimensional GloVe vectors and index build for 1536-dimensional ones)
# ---------------------------------------------------------------------------

def chunk_vectors(X, width: int = 128):
    """Rows of X ([n, D]) zero-padded to C·width coordinates, C = ceil(D/width),
    and cut into chunks: returns [C, n, width] with out[c, i] = coordinates
    c·width .. c·width+width-1 of row i."""
    X = np.asarray(X, np.float64)
    n, D = X.shape
    C = max(1, -(-D // width))
    P = np.zeros((n, C * width))
    P[:, :D] = X
    return np.ascontiguousarray(P.reshape(n, C, width).transpose(1, 0, 2))


def unchunk_vectors(Xc):
    """[C, n, width] → [n, C·width]: chunk c of row i back at coordinates
    c·width ..; the inverse of chunk_vectors on the padded length."""
    Xc = np.asarray(Xc, np.float64)
    C, n, w = Xc.shape
    return np.ascontiguousarray(Xc.transpose(1, 0, 2).reshape(n, C * w))

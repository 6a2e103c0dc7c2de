// Decode attention over a TurboQuant-packed KV cache on gfx950.
//
// Computes, per batch b and query head h (KV head h / G):
//   out = Σ_t softmax_t(scale·⟨q, k̃_t⟩) ṽ_t
// the softmax attention of "I Spent 31 Hours On The Math Behind Turboquant…"
// (onlylabs.fyi), section "KV Cache: The problem", with the full-precision
// query against compressed keys (the asymmetric estimator of "内存厂商的噩梦来了…"
// (wuyi.wiki) section 4.2) and the dequantized vectors
//   k̃ = n (Πᵀ c[idx] + √(π/2)/d · γ · Sᵀ s)   (prod keys; mse keys drop the sketch)
//   ṽ = n Πᵀ c[idx].
// Everything runs in the rotated space: ⟨q, nΠᵀc⟩ = n⟨Πq, c⟩, ⟨q, Sᵀs⟩ = ⟨Sq, s⟩,
// and Σ p n Πᵀc = Πᵀ Σ p n c, so no per-token d×d product is needed.
//
// Three launches on one stream:
//   1. query_prep: q' = Π_K q, q_S = S q per query head, scaled into the log2
//      domain, split into fp16 hi/lo matrix-core B operands.
//   2. attn_split: grid (token split, unit). A unit is one (batch, KV head,
//      group of <= 8 query heads). Each wavefront streams 32-token blocks:
//      codes → fp16 operands through LDS lookup tables, scores on the matrix
//      cores (heads padded to 16 columns), online softmax reduced per
//      wavefront, P·V on the matrix cores into a rotated-space accumulator.
//      The four wavefronts of a workgroup merge in LDS and write one partial
//      (max, sum, acc[128]) per head.
//   3. merge: log-sum-exp combine of the splits, then o = Π_Vᵀ acc / sum.
//
// Precision (rel. L2 vs an fp64 evaluation ~1e-5..1e-4 on Llama-shaped data):
// centroids enter the fp16 tables as c·64·σ with a per-codebook σ in [1, 2)
// chosen by tq_prepare so that they are nearly fp16-exact (≤ 2e-5 relative
// error for ≤ 3-bit codebooks, ≤ 1e-4 for 4-bit ones, whose key table also
// carries the fp16 remainder); q' and q_S are split into fp16 hi + lo, so each
// score takes two (three for 4-bit keys) matrix-core passes; the softmax
// weights are split hi + lo for the two P·V passes; all sums are fp32.
#include <hip/hip_runtime.h>
#include <math.h>

#include "tq.h"
#include "tq_device.h"

int tq_check_quantizer(const tq_quantizer* q);
int tq_device_cus();

namespace tq {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kDecWaves = 4;
constexpr int kBlockTok = 32;            // tokens per wavefront step
constexpr int kMaxHeads = 8;             // query heads per unit
constexpr int kPartStride = 132;         // floats per (unit, split, head) partial: M, L, pad, pad, acc[128]
constexpr int kQFrags = 16;             // q' hi, q' lo, q_S hi, q_S lo × 4 K-steps
constexpr size_t kUnitBytes = kQFrags * 1024 + 256;  // operand fragments + scales

struct Plan {
  int ngroups, units, nsplit, split_len;
  size_t part_off, bytes;
};

inline Plan make_plan(int B, int Hq, int Hkv, int64_t max_ctx) {
  Plan p{};
  const int G = Hq / Hkv;
  p.ngroups = (G + kMaxHeads - 1) / kMaxHeads;
  p.units = B * Hkv * p.ngroups;
  // Aim for ~2048 workgroups over the chip, at least 512 tokens per split.
  int64_t want = (2048 + p.units - 1) / p.units;
  const int64_t max_by_len = (max_ctx + 511) / 512;
  if (want > max_by_len) want = max_by_len;
  if (want < 1) want = 1;
  const int64_t per = (max_ctx + want - 1) / want;
  const int64_t gran = kDecWaves * kBlockTok;
  p.split_len = static_cast<int>((per + gran - 1) / gran * gran);
  p.nsplit = static_cast<int>((max_ctx + p.split_len - 1) / p.split_len);
  p.part_off = (size_t(p.units) * kUnitBytes + 255) / 256 * 256;
  p.bytes = p.part_off + size_t(p.units) * p.nsplit * kMaxHeads * kPartStride * sizeof(float);
  return p;
}

// ---------------------------------------------------------------------------
// 1. Query operands
// ---------------------------------------------------------------------------
struct PrepArgs {
  const float* query;
  const float* rot_k;
  const float* proj;   // null unless the keys carry the sketch
  const PrepHeader* kh;
  float scale;
  int Hq, Hkv, G, ngroups;
  uint8_t* ws;
};

__global__ __launch_bounds__(256) void query_prep_kernel(PrepArgs a) {
  __shared__ float qin[kMaxHeads][kD];
  __shared__ float qp[kMaxHeads][kD];
  __shared__ float qs[kMaxHeads][kD];
  __shared__ float red[2][kMaxHeads][32];
  const int unit = blockIdx.x;
  const int grp = unit % a.ngroups;
  const int kvh = (unit / a.ngroups) % a.Hkv;
  const int b = unit / (a.ngroups * a.Hkv);
  const int h0 = kvh * a.G + grp * kMaxHeads;
  const int gc = min(kMaxHeads, a.G - grp * kMaxHeads);
  const int tid = threadIdx.x;
  for (int e = tid; e < gc * kD; e += 256) qin[e / kD][e % kD] = a.query[(size_t(b) * a.Hq + h0 + e / kD) * kD + e % kD];
  __syncthreads();
  // score = log2(e)·scale·n·(⟨Πq, c⟩ + √(π/2)/d·γ·⟨Sq, s⟩); centroids enter ×64σ.
  const float sq = a.scale * kLog2e / (kCentScale * a.kh->sigma);
  const float ss = a.scale * kLog2e * 1.2533141373155003f / kD;   // √(π/2)/d
  for (int e = tid; e < gc * kD; e += 256) {
    const int c = e / kD, r = e % kD;
    float acc = 0.f, acc2 = 0.f;
    for (int k = 0; k < kD; ++k) acc = fmaf(a.rot_k[r * kD + k], qin[c][k], acc);
    qp[c][r] = acc * sq;
    if (a.proj) {
      for (int k = 0; k < kD; ++k) acc2 = fmaf(a.proj[r * kD + k], qin[c][k], acc2);
      qs[c][r] = acc2 * ss;
    }
  }
  __syncthreads();
  // Per-head power-of-two scale putting max|·| in [2^9, 2^10) for fp16.
  if (tid < 2 * kMaxHeads * 32) {
    const int which = tid / (kMaxHeads * 32), c = (tid / 32) % kMaxHeads, l = tid % 32;
    float m = 0.f;
    if (c < gc && (which == 0 || a.proj))
      for (int r = l; r < kD; r += 32) m = fmaxf(m, fabsf(which ? qs[c][r] : qp[c][r]));
    red[which][c][l] = m;
  }
  __syncthreads();
  __shared__ float scl[2][kMaxHeads];
  if (tid < 2 * kMaxHeads) {
    const int which = tid / kMaxHeads, c = tid % kMaxHeads;
    float m = 0.f;
    for (int l = 0; l < 32; ++l) m = fmaxf(m, red[which][c][l]);
    int ex = 0;
    if (m > 0.f) frexpf(m, &ex);
    scl[which][c] = (m > 0.f) ? ldexpf(1.0f, 10 - ex) : 1.0f;
  }
  __syncthreads();
  uint8_t* blk = a.ws + size_t(unit) * kUnitBytes;
  uint16_t* fr = reinterpret_cast<uint16_t*>(blk);
  // Fragment f, lane l = (n, g), slot j: column n (head), rotated dim 32g + 8(f%4) + j;
  // f/4 = 0: q' hi, 1: q' lo, 2: q_S hi, 3: q_S lo.
  for (int e = tid; e < kQFrags * 64 * 8; e += 256) {
    const int j = e & 7, lane = (e >> 3) & 63, f = e >> 9;
    const int n = lane & 15, g = lane >> 4, s = f & 3;
    const int dim = 32 * g + 8 * s + j;
    uint16_t v = 0;
    if (n < gc) {
      uint16_t hi, lo;
      if (f < 8) {
        split_h(qp[n][dim] * scl[0][n], hi, lo);
        v = (f < 4) ? hi : lo;
      } else if (a.proj) {
        split_h(qs[n][dim] * scl[1][n], hi, lo);
        v = (f < 12) ? hi : lo;
      }
    }
    fr[e] = v;
  }
  float* sc = reinterpret_cast<float*>(blk + kQFrags * 1024);
  if (tid < 32) {
    const int which = tid / 16, c = tid % 16;
    sc[tid] = (c < gc) ? 1.0f / scl[which][c] : 0.f;
  }
}

// ---------------------------------------------------------------------------
// 2. Split attention
// ---------------------------------------------------------------------------
struct AttnArgs {
  const uint8_t* kc;
  const float* kn;
  const uint8_t* kq;
  const float* kg;
  const uint8_t* vc;
  const float* vn;
  const int32_t* ctx_lens;
  int64_t max_ctx;
  const float* kcent;
  const float* vcent;
  const PrepHeader* kh;
  const PrepHeader* vh;
  const uint8_t* ws;
  float* part;
  int Hkv, G, ngroups, nsplit, split_len;
};

// W bits at compile-time bit offset OFF of a little-endian word array.
template <int OFF, int W, int N>
__device__ __forceinline__ uint32_t bits_at(const uint32_t (&w)[N]) {
  constexpr int wi = OFF >> 5, off = OFF & 31;
  constexpr uint32_t mask = (W >= 32) ? 0xffffffffu : ((1u << W) - 1u);
  if constexpr (off + W <= 32) {
    return (w[wi] >> off) & mask;
  } else {
    return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], off) & mask;
  }
}

// Key-code lookup tables. Each entry covers a group of codes (pairs for 3/4
// bits, quads for 2, octets for 1) and holds their fp16 centroids c·64σ
// packed in pairs; 4-bit tables append the fp16 remainders (lo parts).
template <int BK> struct KLut {
  static constexpr bool lo = BK == 4;
  static constexpr int per = BK >= 3 ? 2 : BK == 2 ? 4 : 8;       // codes per entry
  static constexpr int entries = BK == 3 ? 64 : BK >= 1 ? 256 : 0;
  static constexpr int u32_per_entry = (per / 2) * (lo ? 2 : 1);
};

// A operands of K-step s from the lane's 32 key codes (hi; lo for 4 bits).
template <int BK>
__device__ __forceinline__ void key_operands(const uint32_t (&kw)[BK > 0 ? BK : 1], int s,
                                             const uint32_t* lut, u32x4& hi, u32x4& lo) {
  if constexpr (BK == 4) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t e = (kw[s] >> (8 * p)) & 0xffu;
      const u32x2 v = *reinterpret_cast<const u32x2*>(lut + 2 * e);
      hi[p] = v[0];
      lo[p] = v[1];
    }
  } else if constexpr (BK == 3) {
    uint32_t e[4];
    // s is a compile-time constant after unrolling in the caller.
#define TQ_K3(S)                                  \
  if (s == S) {                                   \
    e[0] = bits_at<24 * S + 0, 6>(kw);            \
    e[1] = bits_at<24 * S + 6, 6>(kw);            \
    e[2] = bits_at<24 * S + 12, 6>(kw);           \
    e[3] = bits_at<24 * S + 18, 6>(kw);           \
  }
    TQ_K3(0) TQ_K3(1) TQ_K3(2) TQ_K3(3)
#undef TQ_K3
#pragma unroll
    for (int p = 0; p < 4; ++p) hi[p] = lut[e[p]];
  } else if constexpr (BK == 2) {
    const uint32_t h = (kw[s >> 1] >> (16 * (s & 1))) & 0xffffu;
    const u32x2 q0 = *reinterpret_cast<const u32x2*>(lut + 2 * (h & 0xffu));
    const u32x2 q1 = *reinterpret_cast<const u32x2*>(lut + 2 * (h >> 8));
    hi = u32x4{q0[0], q0[1], q1[0], q1[1]};
  } else if constexpr (BK == 1) {
    const uint32_t e = (kw[0] >> (8 * s)) & 0xffu;
    hi = *reinterpret_cast<const u32x4*>(lut + 4 * e);
  }
}

// Codes of dims 8n..8n+7 of one value vector, right-aligned (8·BV bits).
template <int BV>
__device__ __forceinline__ uint32_t load_vgroup(const uint8_t* vec, int n) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(vec);
  if constexpr (BV == 4) {
    return w[n];
  } else if constexpr (BV == 2) {
    return (w[n >> 1] >> (16 * (n & 1))) & 0xffffu;
  } else if constexpr (BV == 1) {
    return (w[n >> 2] >> (8 * (n & 3))) & 0xffu;
  } else {  // BV == 3: bits 24n .. 24n+23
    const int w0 = (3 * n) >> 2, off = (24 * n) & 31;
    const uint32_t lo = w[w0];
    const uint32_t hi = (off > 8) ? w[w0 + 1] : 0u;
    return __builtin_amdgcn_alignbit(hi, lo, off) & 0xffffffu;
  }
}

template <int BK, bool PROD, int BV>
__global__ __launch_bounds__(kDecWaves * 64) void attn_split_kernel(AttnArgs a) {
  constexpr int KB = BK > 0 ? BK : 1;
  constexpr int kLutK = KLut<BK>::entries * KLut<BK>::u32_per_entry;
  __shared__ uint32_t lut_k[kLutK > 0 ? kLutK : 1] __attribute__((aligned(16)));
  __shared__ u32x4 lut_q[PROD ? 256 : 1];
  __shared__ uint32_t lut_v[1 << (2 * BV)];
  __shared__ float wm[kDecWaves][kMaxHeads], wl[kDecWaves][kMaxHeads], wnv[kDecWaves];
  __shared__ float wacc[kDecWaves][kMaxHeads][kD];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int split = blockIdx.x, unit = blockIdx.y;
  const int grp = unit % a.ngroups;
  const int kvh = (unit / a.ngroups) % a.Hkv;
  const int b = unit / (a.ngroups * a.Hkv);
  const int gc = min(kMaxHeads, a.G - grp * kMaxHeads);

  // ---- lookup tables -------------------------------------------------------
  if constexpr (BK > 0) {
    constexpr int KK = 1 << BK;
    const float ks = kCentScale * a.kh->sigma;
    for (int e = tid; e < KLut<BK>::entries; e += blockDim.x) {
      uint32_t* dst = lut_k + e * KLut<BK>::u32_per_entry;
      constexpr int per = KLut<BK>::per;
      uint16_t hi[8], lo[8];
#pragma unroll
      for (int i = 0; i < per; ++i) {
        const int code = (e >> (BK * i)) & (KK - 1);
        split_h(a.kcent[code] * ks, hi[i], lo[i]);
      }
#pragma unroll
      for (int i = 0; i < per / 2; ++i) {
        dst[i] = uint32_t(hi[2 * i]) | (uint32_t(hi[2 * i + 1]) << 16);
        if constexpr (KLut<BK>::lo) dst[per / 2 + i] = uint32_t(lo[2 * i]) | (uint32_t(lo[2 * i + 1]) << 16);
      }
    }
  }
  if constexpr (PROD) {
    for (int e = tid; e < 256; e += blockDim.x) {
      u32x4 v;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t s0 = ((e >> (2 * k)) & 1) ? 0x3C00u : 0xBC00u;
        const uint32_t s1 = ((e >> (2 * k + 1)) & 1) ? 0x3C00u : 0xBC00u;
        v[k] = s0 | (s1 << 16);
      }
      lut_q[e] = v;
    }
  }
  {
    constexpr int KV = 1 << BV;
    const float vs = kCentScale * a.vh->sigma;
    for (int e = tid; e < KV * KV; e += blockDim.x)
      lut_v[e] = uint32_t(f2h_bits(a.vcent[e & (KV - 1)] * vs)) |
                 (uint32_t(f2h_bits(a.vcent[e >> BV] * vs)) << 16);
  }

  // ---- query operands --------------------------------------------------------
  const uint8_t* blk = a.ws + size_t(unit) * kUnitBytes;
  const u32x4* fr = reinterpret_cast<const u32x4*>(blk);
  u32x4 bqh[4], bql[4], bqs[4], bqsl[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    bqh[s] = fr[s * 64 + lane];
    bql[s] = fr[(4 + s) * 64 + lane];
    if constexpr (PROD) {
      bqs[s] = fr[(8 + s) * 64 + lane];
      bqsl[s] = fr[(12 + s) * 64 + lane];
    }
  }
  const float* scl = reinterpret_cast<const float*>(blk + kQFrags * 1024);
  const float inv_qs = scl[n], inv_qss = scl[16 + n];
  __syncthreads();

  // ---- token range of this wavefront ---------------------------------------
  int64_t L = a.max_ctx;
  if (a.ctx_lens) {
    const int64_t l = a.ctx_lens[b];
    L = l < 0 ? 0 : (l > a.max_ctx ? a.max_ctx : l);
  }
  const int64_t per_wave = a.split_len / kDecWaves;
  const int64_t t_begin = int64_t(split) * a.split_len + wave * per_wave;
  const int64_t t_end = min(t_begin + per_wave, L);
  const int64_t base = (int64_t(b) * a.Hkv + kvh) * a.max_ctx;

  float m_run = -INFINITY, l_run = 0.f, nvs = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t t0 = t_begin; t0 < t_end; t0 += kBlockTok) {
    const int64_t last = L - 1;
    // Key codes of token t0 + 16τ + n, the lane's 32 codes (dims 32g..32g+31).
    uint32_t kw[2][KB];
    uint32_t qw[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      int64_t tk = t0 + 16 * tau + n;
      tk = tk < last ? tk : last;
      if constexpr (BK > 0) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(a.kc + (base + tk) * (16 * BK) + 4 * BK * g);
        if constexpr (BK == 4) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(src);
          kw[tau][0] = v[0]; kw[tau][1] = v[1]; kw[tau][2] = v[2]; kw[tau][3] = v[3];
        } else if constexpr (BK == 2) {
          const u32x2 v = *reinterpret_cast<const u32x2*>(src);
          kw[tau][0] = v[0]; kw[tau][1] = v[1];
        } else {
#pragma unroll
          for (int k = 0; k < BK; ++k) kw[tau][k] = src[k];
        }
      }
      if constexpr (PROD) qw[tau] = *reinterpret_cast<const uint32_t*>(a.kq + (base + tk) * 16 + 4 * g);
    }
    // Per-token scalars for the lane's 8 score slots j = 4τ + i <-> token t0 + 16τ + 4g + i.
    float nk[8], gk[8], nv[8];
    uint32_t cw[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int64_t t = t0 + 16 * (j >> 2) + 4 * g + (j & 3);
      t = t < last ? t : last;
      nk[j] = a.kn[base + t];
      if constexpr (PROD) gk[j] = a.kg[base + t];
      nv[j] = a.vn[base + t];
      cw[j] = load_vgroup<BV>(a.vc + (base + t) * (16 * BV), n);
    }

    // ---- scores: column n = head, rows = 16 tokens of tile τ --------------
    float sc[8];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      f32x4 dm = f32x4{0.f, 0.f, 0.f, 0.f}, dq = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (BK > 0) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          u32x4 ah, al;
          key_operands<BK>(kw[tau], s, lut_k, ah, al);
          dm = mfma(ah, bqh[s], dm);
          dm = mfma(ah, bql[s], dm);
          if constexpr (KLut<BK>::lo) dm = mfma(al, bqh[s], dm);
        }
      }
      if constexpr (PROD) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u32x4 sg = lut_q[(qw[tau] >> (8 * s)) & 0xffu];
          dq = mfma(sg, bqs[s], dq);
          dq = mfma(sg, bqsl[s], dq);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 4 * tau + i;
        float v = dm[i] * inv_qs;
        if constexpr (PROD) v = fmaf(gk[j] * dq[i], inv_qss, v);
        v *= nk[j];
        const int64_t t = t0 + 16 * tau + 4 * g + i;
        sc[j] = (t < t_end) ? v : -INFINITY;
      }
    }

    // ---- online softmax (log2 domain), reduced per wavefront ---------------
    float mloc = sc[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mloc = fmaxf(mloc, sc[j]);
    mloc = max4g(mloc);
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = exp2f(m_run - m_new);
    float p[8], psum = 0.f, nvloc = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = exp2f(sc[j] - m_new);
      psum += p[j];
      nvloc = fmaxf(nvloc, (sc[j] > -INFINITY) ? nv[j] : 0.f);
    }
    l_run = fmaf(l_run, alpha, psum);
    nvloc = max4g(nvloc);
    const float nvs_new = fmaxf(nvs, nvloc);
    const float beta = nvs_new > 0.f ? nvs / nvs_new : 1.f;
    const float inv_nvs = nvs_new > 0.f ? 1.f / nvs_new : 0.f;
    u32x4 pa, pal;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint16_t h0, l0, h1, l1;
      split_h(p[2 * k] * nv[2 * k] * inv_nvs, h0, l0);
      split_h(p[2 * k + 1] * nv[2 * k + 1] * inv_nvs, h1, l1);
      pa[k] = uint32_t(h0) | (uint32_t(h1) << 16);
      pal[k] = uint32_t(l0) | (uint32_t(l1) << 16);
    }
    const float f = alpha * beta;
    if (__any(f != 1.f)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float fi = __shfl(f, 4 * g + i, 64);
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[r][i] *= fi;
      }
    }
    m_run = m_new;
    nvs = nvs_new;

    // ---- P·V: B operand column n = dim 8n + r, rows = token slots ----------
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      u32x4 bv;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t ca = (cw[2 * k] >> (BV * r)) & ((1u << BV) - 1u);
        const uint32_t cb = (cw[2 * k + 1] >> (BV * r)) & ((1u << BV) - 1u);
        bv[k] = lut_v[ca | (cb << BV)];
      }
      acc[r] = mfma(pa, bv, acc[r]);
      acc[r] = mfma(pal, bv, acc[r]);
    }
  }
  l_run = sum4g(l_run);

  // ---- merge the workgroup's wavefronts ------------------------------------
  if (g == 0 && n < kMaxHeads) {
    wm[wave][n] = m_run;
    wl[wave][n] = l_run;
  }
  if (lane == 0) wnv[wave] = nvs;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int head = 4 * g + i;
    if (head < kMaxHeads) {
#pragma unroll
      for (int r = 0; r < 8; ++r) wacc[wave][head][8 * n + r] = acc[r][i];
    }
  }
  __syncthreads();
  float* out = a.part + ((size_t(unit) * a.nsplit + split) * kMaxHeads) * kPartStride;
  for (int e = tid; e < gc * kD; e += blockDim.x) {
    const int head = e / kD, dim = e % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, wm[w][head]);
    float Ls = 0.f, A = 0.f;
    if (M > -INFINITY) {
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        const float fw = exp2f(wm[w][head] - M);
        Ls = fmaf(fw, wl[w][head], Ls);
        A = fmaf(fw * wnv[w], wacc[w][head][dim], A);
      }
    }
    float* o = out + head * kPartStride;
    o[4 + dim] = A;
    if (dim == 0) {
      o[0] = M;
      o[1] = Ls;
    }
  }
}

// ---------------------------------------------------------------------------
// 3. Merge splits and rotate back
// ---------------------------------------------------------------------------
struct MergeArgs {
  const float* part;
  const float* rot_v;
  const PrepHeader* vh;
  float* out;
  int Hq, Hkv, G, ngroups, nsplit;
};

__global__ __launch_bounds__(kD) void merge_kernel(MergeArgs a) {
  __shared__ float orot[kD];
  const int bh = blockIdx.x;
  const int h = bh % a.Hq, b = bh / a.Hq;
  const int kvh = h / a.G, hin = h % a.G;
  const int unit = (b * a.Hkv + kvh) * a.ngroups + hin / kMaxHeads;
  const int slot = hin % kMaxHeads;
  const int dim = threadIdx.x;
  const float* p = a.part + (size_t(unit) * a.nsplit * kMaxHeads + slot) * kPartStride;
  const size_t stride = size_t(kMaxHeads) * kPartStride;
  float M = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, p[s * stride]);
  float Ls = 0.f, A = 0.f;
  if (M > -INFINITY) {
    for (int s = 0; s < a.nsplit; ++s) {
      const float* ps = p + s * stride;
      const float f = exp2f(ps[0] - M);
      Ls = fmaf(f, ps[1], Ls);
      A = fmaf(f, ps[4 + dim], A);
    }
  }
  orot[dim] = (Ls > 0.f) ? A / (Ls * kCentScale * a.vh->sigma) : 0.f;
  __syncthreads();
  float o = 0.f;
  for (int j = 0; j < kD; ++j) o = fmaf(a.rot_v[j * kD + dim], orot[j], o);
  a.out[size_t(bh) * kD + dim] = o;
}

template <int BK, bool PROD, int BV>
hipError_t launch_attn_t(const AttnArgs& a, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((attn_split_kernel<BK, PROD, BV>), grid, dim3(kDecWaves * 64), 0, st, a);
  return hipGetLastError();
}

template <int BK, bool PROD>
hipError_t launch_attn_bv(const AttnArgs& a, int bv, dim3 grid, hipStream_t st) {
  switch (bv) {
    case 1: return launch_attn_t<BK, PROD, 1>(a, grid, st);
    case 2: return launch_attn_t<BK, PROD, 2>(a, grid, st);
    case 3: return launch_attn_t<BK, PROD, 3>(a, grid, st);
    default: return launch_attn_t<BK, PROD, 4>(a, grid, st);
  }
}

}  // namespace tq

using namespace tq;

extern "C" size_t tq_attn_decode_workspace(int B, int Hq, int Hkv, int64_t max_ctx) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_ctx < 1) return 0;
  return make_plan(B, Hq, Hkv, max_ctx).bytes;
}

namespace {

int decode_call(int phase, const tq_quantizer* kq, const tq_quantizer* vq, const float* query, int B,
                int Hq, int Hkv, const int32_t* ctx_lens, int64_t max_ctx, const tq_packed* k_cache,
                const tq_packed* v_cache, float scale, float* out, void* workspace, size_t ws_bytes,
                void* stream) {
  if (phase < 0 || phase > 3) return TQ_ERR_INVALID_ARG;
  int st = tq_check_quantizer(kq);
  if (st != TQ_OK) return st;
  st = tq_check_quantizer(vq);
  if (st != TQ_OK) return st;
  if (vq->variant != TQ_MSE) return TQ_ERR_UNSUPPORTED;
  if (query == nullptr || out == nullptr || k_cache == nullptr || v_cache == nullptr || workspace == nullptr)
    return TQ_ERR_INVALID_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_ctx < 1) return TQ_ERR_INVALID_ARG;
  const bool prod = kq->variant == TQ_PROD;
  const int bk = prod ? kq->bits - 1 : kq->bits;
  if (k_cache->norms == nullptr || (bk > 0 && k_cache->codes == nullptr)) return TQ_ERR_INVALID_ARG;
  if (prod && (k_cache->qjl == nullptr || k_cache->gammas == nullptr)) return TQ_ERR_INVALID_ARG;
  if (v_cache->norms == nullptr || v_cache->codes == nullptr) return TQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(k_cache->codes) | reinterpret_cast<uintptr_t>(v_cache->codes) |
       reinterpret_cast<uintptr_t>(prod ? k_cache->qjl : nullptr)) % 16 != 0)
    return TQ_ERR_INVALID_ARG;
  const Plan p = make_plan(B, Hq, Hkv, max_ctx);
  if (ws_bytes < p.bytes || reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return TQ_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const int G = Hq / Hkv;
  float* part = reinterpret_cast<float*>(ws + p.part_off);

  if (phase == 0 || phase == 1) {
    PrepArgs pa{query, kq->rot, prod ? kq->proj : nullptr, static_cast<const PrepHeader*>(kq->prep), scale,
                Hq, Hkv, G, p.ngroups, ws};
    hipLaunchKernelGGL(query_prep_kernel, dim3(p.units), dim3(256), 0, s, pa);
    if (hipGetLastError() != hipSuccess) return TQ_ERR_HIP;
  }
  if (phase == 0 || phase == 2) {
    AttnArgs aa;
    aa.kc = k_cache->codes;
    aa.kn = k_cache->norms;
    aa.kq = k_cache->qjl;
    aa.kg = k_cache->gammas;
    aa.vc = v_cache->codes;
    aa.vn = v_cache->norms;
    aa.ctx_lens = ctx_lens;
    aa.max_ctx = max_ctx;
    aa.kcent = kq->centroids;
    aa.vcent = vq->centroids;
    aa.kh = static_cast<const PrepHeader*>(kq->prep);
    aa.vh = static_cast<const PrepHeader*>(vq->prep);
    aa.ws = ws;
    aa.part = part;
    aa.Hkv = Hkv;
    aa.G = G;
    aa.ngroups = p.ngroups;
    aa.nsplit = p.nsplit;
    aa.split_len = p.split_len;
    const dim3 grid(p.nsplit, p.units);
    const int bv = vq->bits;
    hipError_t e;
    if (!prod) {
      switch (bk) {
        case 1: e = launch_attn_bv<1, false>(aa, bv, grid, s); break;
        case 2: e = launch_attn_bv<2, false>(aa, bv, grid, s); break;
        case 3: e = launch_attn_bv<3, false>(aa, bv, grid, s); break;
        default: e = launch_attn_bv<4, false>(aa, bv, grid, s); break;
      }
    } else {
      switch (bk) {
        case 0: e = launch_attn_bv<0, true>(aa, bv, grid, s); break;
        case 1: e = launch_attn_bv<1, true>(aa, bv, grid, s); break;
        case 2: e = launch_attn_bv<2, true>(aa, bv, grid, s); break;
        default: e = launch_attn_bv<3, true>(aa, bv, grid, s); break;
      }
    }
    if (e != hipSuccess) return TQ_ERR_HIP;
  }
  if (phase == 0 || phase == 3) {
    MergeArgs ma{part, vq->rot, static_cast<const PrepHeader*>(vq->prep), out, Hq, Hkv, G, p.ngroups, p.nsplit};
    hipLaunchKernelGGL(merge_kernel, dim3(B * Hq), dim3(kD), 0, s, ma);
    if (hipGetLastError() != hipSuccess) return TQ_ERR_HIP;
  }
  return TQ_OK;
}

}  // namespace

extern "C" int tq_attn_decode(const tq_quantizer* kq, const tq_quantizer* vq, const float* query,
                              int B, int Hq, int Hkv, const int32_t* ctx_lens, int64_t max_ctx,
                              const tq_packed* k_cache, const tq_packed* v_cache, float scale,
                              float* out, void* workspace, size_t ws_bytes, void* stream) {
  return decode_call(0, kq, vq, query, B, Hq, Hkv, ctx_lens, max_ctx, k_cache, v_cache, scale, out,
                     workspace, ws_bytes, stream);
}

extern "C" int tq_attn_decode_phase(int phase, const tq_quantizer* kq, const tq_quantizer* vq,
                                    const float* query, int B, int Hq, int Hkv, const int32_t* ctx_lens,
                                    int64_t max_ctx, const tq_packed* k_cache, const tq_packed* v_cache,
                                    float scale, float* out, void* workspace, size_t ws_bytes,
                                    void* stream) {
  if (phase < 1 || phase > 3) return TQ_ERR_INVALID_ARG;
  return decode_call(phase, kq, vq, query, B, Hq, Hkv, ctx_lens, max_ctx, k_cache, v_cache, scale, out,
                     workspace, ws_bytes, stream);
}

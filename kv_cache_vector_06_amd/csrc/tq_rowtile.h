// Row-tile-parallel encoder for launches far too small to fill the chip (a
// decode step's one-token append; any encode of a few hundred rows).
//
// What it computes is the encoder of "TurboQuant của Google…" (omelet.tech),
// sections "Trick đầu tiên…" (y = Π·x/‖x‖) and "Lloyd-Max quantizer…" (the
// nearest-centroid index, LSB-first packed), plus for prod its QJL section
// (residual, γ = ‖r‖, 1-bit sketch sign(S·r)), exactly as the full-size encoder
// does it.
//
// How. A workgroup of 8 wavefronts takes one tile of 16 rows. Wavefront t
// computes output row tile t only (16 of the 128 rotated coordinates of every
// row), from its 8 KiB share of the prepared fragments read straight from
// memory instead of staging all 64–128 KiB of them in LDS first; the tile's
// pieces (code bits, residual operands, sketch bits) meet in LDS. Every value
// is formed by the same operations in the same order as in the full-size
// encoder (matrix-core passes per K-step, the scaled bit-pattern compares, the
// residual sum over coordinates 0..127 of a lane group), so the two encoders
// give bit-identical results.
#pragma once

#include "tq_device.h"

namespace tq {

constexpr int kRowWaves = 8;   // one wavefront per output row tile

// LDS exchange area of a row-tile workgroup (23.5 KiB).
struct RowXchg {
  u32x2 b[2][8][64];      // fp16 hi (0) / lo (1) B-operand dwords from row tile t
  float racc[8][4][64];   // S·(y - c) of row tile t, element j
  uint32_t piece[8][64];  // code bits of row tile t
  uint32_t sbits[8][64];  // sketch bits of row tile t
  float red[2][8][16];    // per-(row tile, column) maxima, two rounds
  float bmax[8][64];      // per-(row tile, lane) maxima (query prep: sketch operand blocks)
};

struct RowEncArgs {
  const void* x;
  int64_t n;
  int64_t stride;          // elements between rows
  int f32in;               // 1: float32 rows, 0: bfloat16 rows
  int bm;                  // Lloyd-Max bits (0 for the 1-bit prod quantizer)
  int prod;
  uint8_t* codes;
  float* norms;
  uint8_t* qjl;
  float* gammas;
  const u32x4* frags;      // 16Π fragments, then (prod) S' = S·Πᵀ
  const float* centroids;
  const float* boundaries;
  const int64_t* slot;     // output slot of each row, or null
  // Append mode (slot == null, append != 0): row r = b·hkv + h goes to slot
  // r·max_ctx + len_b - 1 with len_b = lens[b] (max_ctx when lens is null),
  // and is not written unless 1 <= len_b <= max_ctx.
  const int32_t* lens;
  int64_t max_ctx;
  int hkv;
  int append;
};

// Encode 16-row tile `tile`; every wavefront of the workgroup must call it.
__device__ __forceinline__ void row_encode(const RowEncArgs& a, int64_t tile, RowXchg& X) {
  const int lane = threadIdx.x & 63;
  const int t = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int64_t rowi = tile * 16 + n;
  bool valid = rowi < a.n;
  const int64_t row = valid ? rowi : a.n - 1;
  int64_t vec = row;
  if (a.slot != nullptr) {
    vec = a.slot[row];
  } else if (a.append) {
    const int64_t len = a.lens != nullptr ? int64_t(a.lens[row / a.hkv]) : a.max_ctx;
    valid = valid && len >= 1 && len <= a.max_ctx;
    vec = row * a.max_ctx + (len - 1);
  }

  // The header's rotation scale and the codebook, read up front through the
  // scalar unit (uniform addresses), so that their latency overlaps the
  // fragment loads instead of following the products.
  const uint32_t K2 = a.bm > 0 ? (1u << a.bm) / 2 : 0u;
  const float rot_scale =
      scalar_load(&reinterpret_cast<const PrepHeader*>(reinterpret_cast<const uint8_t*>(a.frags) - kPrepHeaderBytes)->rot_scale);
  float tb[8], cb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    tb[j] = (j >= 1 && uint32_t(j) < K2) ? scalar_load(a.boundaries + (K2 - 1 + j)) : 0.f;
    cb[j] = uint32_t(j) < K2 ? scalar_load(a.centroids + (K2 + j)) : 0.f;
  }
  // This wavefront's fragments: 16Π (hi, lo) and S' (hi, lo) of row tile t.
  u32x4 rh[4], rl[4], ph[4], pl[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    rh[s] = a.frags[frag_index(0, t, s) * 64 + lane];
    rl[s] = a.frags[frag_index(1, t, s) * 64 + lane];
  }
  if (a.prod) {
    const u32x4* fp = a.frags + kFragsPerSet * 64;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      ph[s] = fp[frag_index(0, t, s) * 64 + lane];
      pl[s] = fp[frag_index(1, t, s) * 64 + lane];
    }
  }
  // Row n, columns 32s + 8g + j in slot 8s + j.
  float xv[32];
  if (!a.f32in) {
    const uint16_t* xr = static_cast<const uint16_t*>(a.x) + row * a.stride + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 r = *reinterpret_cast<const u32x4*>(xr + 32 * s);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        xv[8 * s + 2 * k] = bf16_to_f32(r[k] & 0xffffu);
        xv[8 * s + 2 * k + 1] = bf16_to_f32(r[k] >> 16);
      }
    }
  } else {
    const float* xr = static_cast<const float*>(a.x) + row * a.stride + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(xr + 32 * s);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(xr + 32 * s + 4);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        xv[8 * s + k] = w0[k];
        xv[8 * s + 4 + k] = w1[k];
      }
    }
  }
  // Norm and the fp16 form of the row, as it is or scaled by 2^-e
  // (row_exponent, the same choice as the full-size encoder's).
  float ss = 0.f;
  int ex = 0;
  if (!a.f32in) {
    ss = row_ss<false>(xv);
    ex = row_exponent<false>(xv, ss);
  } else {
    ex = row_exponent<true>(xv, ss);
  }
  const float rs = sqrtf(ss);
  const float nrm = ldexpf(rs, ex);
  u32x4 bx[4], bxl[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (!a.f32in) {
        bx[s][k] = bf16_row_pair(xv[8 * s + 2 * k], xv[8 * s + 2 * k + 1]);
        bxl[s][k] = 0u;
      } else {
        uint16_t h0, l0, h1, l1;
        split_h(xv[8 * s + 2 * k], h0, l0);
        split_h(xv[8 * s + 2 * k + 1], h1, l1);
        bx[s][k] = uint32_t(h0) | (uint32_t(h1) << 16);
        bxl[s][k] = uint32_t(l0) | (uint32_t(l1) << 16);
      }
    }
  // acc = S·y for rotated coordinates 32g + 4t + j, S = rot_scale·‖x‖·2^-e.
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    acc = mfma(rh[s], bx[s], acc);
    acc = mfma(rl[s], bx[s], acc);
    if (a.f32in) acc = mfma(rh[s], bxl[s], acc);
  }

  // Scaled codebook: T[j] = bits(S·t_j) for 1 <= j < K/2 (all ones above,
  // never below a magnitude), cs[m] = S·(centroid magnitude m).
  const float S = (rs > 0.f) ? rot_scale * rs : 1.0f;
  const float up = 1.0f / S;
  uint32_t T[8];
  float cs[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    T[j] = (j >= 1 && uint32_t(j) < K2) ? __builtin_bit_cast(uint32_t, tb[j] * S) : 0xffffffffu;
    cs[j] = uint32_t(j) < K2 ? cb[j] * S : 0.f;
  }
  // code = #{j >= 1 : T_j < |acc|} (|acc| + 1 ulp when acc <= 0: ties go to
  // the lower index), then m ^ K/2 or m ^ (K/2 - 1).
  // (bit-cast the whole vector: a bit cast of one vector element reads element 0)
  const u32x4 accb = __builtin_bit_cast(u32x4, acc);
  uint32_t piece = 0u;
  float racc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t vb = accb[j];
    const bool pos = static_cast<int32_t>(vb) > 0;
    const uint32_t ab = (vb & 0x7fffffffu) + (pos ? 0u : 1u);
    uint32_t m = 0u;
#pragma unroll
    for (int k = 1; k < 8; ++k) m += ab > T[k] ? 1u : 0u;
    piece |= (m ^ (pos ? K2 : K2 - 1u)) << (j * a.bm);
    float c = 0.f;
    if (a.bm > 0) {
      c = cs[0];
#pragma unroll
      for (int k = 1; k < 8; ++k) c = (m == uint32_t(k)) ? cs[k] : c;
      c = pos ? c : -c;
    }
    racc[j] = acc[j] - c;   // S·(y - c)
  }
  X.piece[t][lane] = piece;
  if (a.prod) {
    const float rsc = up * kResScale;
    uint16_t h[4], l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      X.racc[t][j][lane] = racc[j];
      split_h(racc[j] * rsc, h[j], l[j]);   // 64·(y - c)
    }
    X.b[0][t][lane] = u32x2{uint32_t(h[0]) | (uint32_t(h[1]) << 16), uint32_t(h[2]) | (uint32_t(h[3]) << 16)};
    X.b[1][t][lane] = u32x2{uint32_t(l[0]) | (uint32_t(l[1]) << 16), uint32_t(l[2]) | (uint32_t(l[3]) << 16)};
  }
  __syncthreads();

  if (t == 0) {
    // Codes of lane group g: code q = 4t' + j at bit q·bm of a 32·bm-bit word run.
    if (a.bm > 0 && valid) {
      uint64_t lo = 0u, hi = 0u;
      const int w = 4 * a.bm;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const uint64_t p = X.piece[tt][lane];
        const int off = tt * w;
        if (off < 64) {
          lo |= p << off;
          if (off + w > 64) hi |= p >> (64 - off);
        } else {
          hi |= p << (off - 64);
        }
      }
      uint32_t* dst = reinterpret_cast<uint32_t*>(a.codes + vec * (16 * a.bm) + 4 * a.bm * g);
      for (int k = 0; k < a.bm; ++k) dst[k] = static_cast<uint32_t>(k < 2 ? lo >> (32 * k) : hi >> (32 * (k - 2)));
    }
    if (valid && g == 0) a.norms[vec] = nrm;
  }
  if (!a.prod) return;

  // Sketch z = S'·(64(y - c)) for row tile t, from the whole residual.
  u32x4 bh[4], bl[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const u32x2 e0 = X.b[0][2 * s][lane], e1 = X.b[0][2 * s + 1][lane];
    const u32x2 f0 = X.b[1][2 * s][lane], f1 = X.b[1][2 * s + 1][lane];
    bh[s] = u32x4{e0[0], e0[1], e1[0], e1[1]};
    bl[s] = u32x4{f0[0], f0[1], f1[0], f1[1]};
  }
  f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    z = mfma(ph[s], bh[s], z);
    z = mfma(pl[s], bh[s], z);
    z = mfma(ph[s], bl[s], z);
  }
  uint32_t sb = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) sb |= uint32_t(z[j] >= 0.f) << j;
  X.sbits[t][lane] = sb;
  if (t == 1) {
    // ‖S·(y - c)‖² summed over the lane group's coordinates in order, then
    // over the four groups.
    float r2 = 0.f;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
#pragma unroll
      for (int j = 0; j < 4; ++j) r2 = fmaf(X.racc[tt][j][lane], X.racc[tt][j][lane], r2);
    r2 = sum4g(r2);
    if (valid && g == 0) a.gammas[vec] = sqrtf(r2) * up;
  }
  __syncthreads();
  if (t == 0 && valid) {
    uint32_t word = 0u;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) word |= X.sbits[tt][lane] << (4 * tt);
    *reinterpret_cast<uint32_t*>(a.qjl + vec * 16 + 4 * g) = word;
  }
}

}  // namespace tq

// TurboQuant encoder on gfx950: norm → rotation on the matrix cores →
// Lloyd-Max nearest-centroid codes → LSB-first bit packing; the prod variant
// adds the residual, its norm γ and the 1-bit QJL sketch sign(S·r).
//
// Method: "The Distortion Guarantee — How Good Is This?" ("rotate, quantize,
// done"); "TurboQuant của Google…" (omelet.tech) sections "Trick đầu tiên:
// xoay ngẫu nhiên trước khi nén" (Π from QR of a Gaussian, y = Π·u) and
// "Lloyd-Max quantizer: chia bucket đúng chỗ" (store the nearest-centroid
// index), and its QJL section ((b-1)-bit quantizer, residual, 1-bit sketch);
// "内存厂商的噩梦来了…" (wuyi.wiki) sections 4.2-4.3.
//
// Precision. A code may differ from an exact-arithmetic encoder only where the
// rotated coordinate lies within ~1e-7 of a boundary, so Π·x needs fp32-level
// accuracy. The rotation runs on the fp16 matrix cores with Π split into two
// fp16 parts (hi + lo ≈ 22-bit mantissa) and x converted exactly: bf16 inputs
// fit fp16 after scaling the vector by a power of two (2^-e, max|x| = m·2^e)
// so that every component is below 1 in magnitude; fp32 inputs are split into
// two fp16 parts as well. Products of fp16 values are exact in the fp32
// accumulator. The prod sketch uses S' = S·Πᵀ on the rotated residual
// r̂ = y - c[idx] (S'·r̂ = S·r exactly), with three fp16-split passes.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "tq.h"
#include "tq_device.h"
#include "tq_rowtile.h"

namespace tq {


// ---------------------------------------------------------------------------
// Outlier-channel split ("TurboQuant của Google…" (omelet.tech), section
// "Thực nghiệm: 3.5 bit…"): the two groups' rotations as one d×d matrix.
// Position p with p mod 8 < 2 is outlier row k = 2(p/8) + p mod 8 and holds
// Π_o[k][j] at the j-th outlier channel; another position p is regular row
// k = 6(p/8) + p mod 8 - 2 and holds Π_r[k][j] at the j-th regular channel
// (increasing order). Every other entry is zero. One workgroup per row.
// ---------------------------------------------------------------------------
struct SplitChannels {
  // column c of the block matrix: j < 32 when c is the j-th outlier channel
  // (Π_o's column j), 32 + j when c is the j-th regular channel (Π_r's column j)
  int32_t slot[128];
};

__global__ __launch_bounds__(128) void split_rotation_kernel(const float* __restrict__ rot_o,
                                                             const float* __restrict__ rot_r, SplitChannels ch,
                                                             float* __restrict__ out) {
  const int p = blockIdx.x, col = threadIdx.x;
  const int j = ch.slot[col];
  float v = 0.f;
  if ((p & 7) < 2) {
    if (j < 32) v = rot_o[(2 * (p >> 3) + (p & 7)) * 32 + j];
  } else {
    if (j >= 32) v = rot_r[(6 * (p >> 3) + (p & 7) - 2) * 96 + (j - 32)];
  }
  out[p * kD + col] = v;
}

// ---------------------------------------------------------------------------
// tq_prepare: fragment the rotation (and S' = S·Πᵀ) into matrix-core A operands
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void prepare_kernel(const float* __restrict__ rot,
                                                       const float* __restrict__ proj,
                                                       const float* __restrict__ centroids, int bm,
                                                       int hadamard, const float* __restrict__ centroids_o,
                                                       uint8_t* __restrict__ prep_base) {
  __shared__ float red[1024];
  __shared__ int redi[1024];
  const int tid = threadIdx.x;
  // Centroid scale σ in [1, 2): the centroid magnitudes times 64σ are as close
  // to fp16 values as any σ on a 2^-18 grid makes them (max relative error
  // over the magnitudes, smallest σ on ties).
  {
    const int half = bm > 0 ? (1 << bm) / 2 : 0;
    float best = INFINITY;
    int bi = 0;
    for (int k = tid; k < (1 << 18); k += 1024) {
      const float sg = 1.0f + float(k) * (1.0f / (1 << 18));
      float err = 0.f;
      for (int m = 0; m < half; ++m) {
        const float v = centroids[half + m] * kCentScale * sg;
        if (v > 0.f) err = fmaxf(err, fabsf(h2f(f2h_bits(v)) - v) / v);
      }
      if (centroids_o != nullptr) {   // split: the outlier codebook (bm + 1 bits) shares σ
        const int ho = 1 << bm;
        for (int m = 0; m < ho; ++m) {
          const float v = centroids_o[ho + m] * kCentScale * sg;
          if (v > 0.f) err = fmaxf(err, fabsf(h2f(f2h_bits(v)) - v) / v);
        }
      }
      if (err < best) {
        best = err;
        bi = k;
      }
    }
    red[tid] = best;
    redi[tid] = bi;
    __syncthreads();
    for (int w = 512; w > 0; w >>= 1) {
      if (tid < w && (red[tid + w] < red[tid] || (red[tid + w] == red[tid] && redi[tid + w] < redi[tid]))) {
        red[tid] = red[tid + w];
        redi[tid] = redi[tid + w];
      }
      __syncthreads();
    }
    if (tid == 0) {
      PrepHeader* h = reinterpret_cast<PrepHeader*>(prep_base);
      h->sigma = 1.0f + float(redi[0]) * (1.0f / (1 << 18));
      h->sigma_err = red[0];
      h->sp_scale = 0.f;
      h->rot_scale = hadamard ? sqrtf(float(kD)) : kRotScale;
      for (int w = 0; w < 4; ++w) h->omask[w] = 0u;
    }
    __syncthreads();
  }
  if (centroids_o != nullptr) {
    // raw channel c is an outlier channel when its column of Π has its (unit)
    // weight in the outlier rows p mod 8 < 2
    __shared__ uint32_t om[4];
    if (tid < 4) om[tid] = 0u;
    __syncthreads();
    if (tid < kD) {
      float e = 0.f;
      for (int p = 0; p < kD; ++p)
        if ((p & 7) < 2) e = fmaf(rot[p * kD + tid], rot[p * kD + tid], e);
      if (e > 0.5f) atomicOr(&om[tid >> 5], 1u << (tid & 31));
    }
    __syncthreads();
    if (tid < 4) reinterpret_cast<PrepHeader*>(prep_base)->omask[tid] = om[tid];
  }
  uint16_t* prep = reinterpret_cast<uint16_t*>(prep_base + kPrepHeaderBytes);
  // Rotation fragments: A(t, s)[lane (i, g)][j] = rot_scale·Π[out_row(t,i)][32s + 8g + j]:
  // the fp16 hi/lo split of 16Π, or for a randomized Hadamard Π = H·diag(s)/√d
  // the exact ±1 entries of H·diag(s) (the signs of Π's entries) with zero lo parts.
  for (int e = tid; e < 8 * 4 * 64 * 8; e += 1024) {
    const int j = e & 7, lane = (e >> 3) & 63, s = (e >> 9) & 3, t = e >> 11;
    const int i = lane & 15, g = lane >> 4;
    const float r = rot[out_row(t, i) * kD + 32 * s + 8 * g + j];
    uint16_t hi, lo;
    if (hadamard) {
      hi = r > 0.f ? 0x3c00u : r < 0.f ? 0xbc00u : 0u;
      lo = 0u;
    } else {
      split_h(kRotScale * r, hi, lo);
    }
    prep[(frag_index(0, t, s) * 64 + lane) * 8 + j] = hi;
    prep[(frag_index(1, t, s) * 64 + lane) * 8 + j] = lo;
  }
  if (proj == nullptr) return;
  // S'[a][c] = Σ_k S[a][k] Π[c][k] in double; scaled by a power of two so that
  // max|S'| lands in [8, 16).
  auto sprime = [&](int a, int c) {
    double acc = 0.0;
    for (int k = 0; k < kD; ++k) acc += double(proj[a * kD + k]) * double(rot[c * kD + k]);
    return acc;
  };
  float mx = 0.f;
  for (int e = tid; e < kD * kD; e += 1024) mx = fmaxf(mx, fabsf(float(sprime(e / kD, e % kD))));
  red[tid] = mx;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  mx = red[0];
  int ex = 0;
  if (mx > 0.f) frexpf(mx, &ex);   // mx = m·2^ex, m in [0.5, 1)
  const double sc = ldexp(1.0, 4 - ex);
  uint16_t* pp = prep + kSetBytes / 2;
  // A(t, s)[lane (i, g)][j] = S'[out_row(t,i)][32g + 8s + j] (the rotated residual
  // columns a lane group holds itself).
  for (int e = tid; e < 8 * 4 * 64 * 8; e += 1024) {
    const int j = e & 7, lane = (e >> 3) & 63, s = (e >> 9) & 3, t = e >> 11;
    const int i = lane & 15, g = lane >> 4;
    const float v = float(sc * sprime(out_row(t, i), 32 * g + 8 * s + j));
    uint16_t hi, lo;
    split_h(v, hi, lo);
    pp[(frag_index(0, t, s) * 64 + lane) * 8 + j] = hi;
    pp[(frag_index(1, t, s) * 64 + lane) * 8 + j] = lo;
  }
  if (tid == 0) reinterpret_cast<PrepHeader*>(prep_base)->sp_scale = float(sc);
}

// ---------------------------------------------------------------------------
// Encode kernel
// ---------------------------------------------------------------------------
#define TQ_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// Copy the 64 KiB fragment set at `src` (and the next one, when `dst2` is not
// null) to LDS: wavefront w of the workgroup issues chunks w, w + W, ... of
// 64 × 16 bytes, then every load is waited for and the workgroup synchronises.
__device__ __forceinline__ void stage_frags(const u32x4* src, u32x4* dst, u32x4* dst2, int tid) {
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = __builtin_amdgcn_readfirstlane(static_cast<int>(blockDim.x) >> 6);
  constexpr int chunks = kFragsPerSet;   // 64 × 64 × 16 B = 64 KiB
  for (int c = wave; c < chunks; c += nw) {
    __builtin_amdgcn_global_load_lds(src + c * 64 + lane, TQ_LDS(dst + c * 64), 16, 0, 0);
    if (dst2 != nullptr)
      __builtin_amdgcn_global_load_lds(src + (chunks + c) * 64 + lane, TQ_LDS(dst2 + c * 64), 16, 0, 0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}
struct EncodeArgs {
  const void* x;
  int64_t n;
  int64_t stride;       // elements between rows
  uint8_t* codes;
  float* norms;
  uint8_t* qjl;
  float* gammas;
  const u32x4* prep;
  const float* centroids;
  const float* boundaries;
  const int64_t* slot;  // output slot of each row, or null for slot = row
  const float* centroids_o;   // split: the outlier group's codebook
  const float* boundaries_o;
  // Append mode of the split encoder (slot == null, append != 0): row
  // r = b·hkv + h goes to slot r·max_ctx + lens[b] - 1 (max_ctx when lens is
  // null) and is not written unless 1 <= lens[b] <= max_ctx.
  const int32_t* lens;
  int64_t max_ctx;
  int hkv;
  int append;
};

constexpr int kEncWaves = 8;

// Thresholds of an antisymmetric codebook with K = 2^BM levels, held in
// scalars: tp[j] = boundaries[K/2-1+j] (tp[0] = 0) and the centroid
// magnitudes cm[m] = centroids[K/2+m].
struct Book {
  float t1, t2, t3, t4, t5, t6, t7;
  float c0, c1, c2, c3, c4, c5, c6, c7;
};

template <int BM>
__device__ __forceinline__ Book load_book(const float* centroids, const float* boundaries) {
  constexpr int K = 1 << BM;
  Book bk{};
  if constexpr (BM >= 1) {
    const float* tb = boundaries + (K / 2 - 1);
    const float* cb = centroids + K / 2;
    bk.c0 = cb[0];
    if constexpr (K / 2 > 1) { bk.t1 = tb[1]; bk.c1 = cb[1]; }
    if constexpr (K / 2 > 2) { bk.t2 = tb[2]; bk.t3 = tb[3]; bk.c2 = cb[2]; bk.c3 = cb[3]; }
    if constexpr (K / 2 > 4) {
      bk.t4 = tb[4]; bk.t5 = tb[5]; bk.t6 = tb[6]; bk.t7 = tb[7];
      bk.c4 = cb[4]; bk.c5 = cb[5]; bk.c6 = cb[6]; bk.c7 = cb[7];
    }
  }
  return bk;
}

// Nearest-centroid code of y: idx = #{i : t_i < y}. With a = |y|:
//   y > 0:  idx = K/2 + #{j >= 1 : tp[j] <  a}
//   y <= 0: idx = K/2 - 1 - #{j >= 1 : tp[j] <= a}
// and "tp <= a" is "tp < nextup(a)" on floats. Also returns the magnitude
// index m (the centroid is +cm[m] when y > 0, -cm[m] otherwise).
template <int BM>
__device__ __forceinline__ uint32_t quantize(float y, const Book& bk, int& m, bool& pos) {
  constexpr int K = 1 << BM;
  pos = y > 0.f;
  float a = fabsf(y);
  a = pos ? a : __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, a) + 1u);
  m = 0;
  if constexpr (BM == 2) {
    m = a > bk.t1;
  } else if constexpr (BM == 3) {
    const int b1 = a > bk.t2;
    const float th = b1 ? bk.t3 : bk.t1;
    m = 2 * b1 + (a > th);
  } else if constexpr (BM == 4) {
    const int b2 = a > bk.t4;
    const float t1 = b2 ? bk.t6 : bk.t2;
    const int b1 = a > t1;
    const float thi = b1 ? bk.t7 : bk.t5;
    const float tlo = b1 ? bk.t3 : bk.t1;
    const float t0 = b2 ? thi : tlo;
    m = 4 * b2 + 2 * b1 + (a > t0);
  }
  if constexpr (BM == 0) return 0u;
  return pos ? uint32_t(K / 2 + m) : uint32_t(K / 2 - 1 - m);
}

// The same search on the matrix-core output acc = S·y (S > 0, one per
// vector), against thresholds scaled by S and compared as bit patterns
// (non-negative floats order like their bit patterns): with a = |acc| and
// m = #{j >= 1 : T_j < a} (acc > 0) or #{j >= 1 : T_j <= a} (acc <= 0, ties
// to the lower index; "T <= a" is "T < a + 1 ulp"), the code is K/2 + m or
// K/2 - 1 - m, i.e. m ^ K/2 or m ^ (K/2 - 1).
struct ScaledBook {
  uint32_t t[8];   // bits of S·t_j, j = 1 .. K/2 - 1
  float c[8];      // S·(centroid magnitudes)
};

template <int BM>
__device__ __forceinline__ uint32_t quantize_scaled(float acc, const ScaledBook& sb, uint32_t& m, bool& pos) {
  constexpr uint32_t K2 = (1u << BM) / 2;
  const uint32_t vb = __builtin_bit_cast(uint32_t, acc);
  pos = static_cast<int32_t>(vb) > 0;
  const uint32_t ab = (vb & 0x7fffffffu) + (pos ? 0u : 1u);
  m = 0u;
  if constexpr (BM == 2) {
    m = ab > sb.t[1];
  } else if constexpr (BM == 3) {
    const uint32_t c1 = ab > sb.t[2];
    const uint32_t th = c1 ? sb.t[3] : sb.t[1];
    m = c1 + c1 + (ab > th);
  } else if constexpr (BM == 4) {
    const uint32_t c2 = ab > sb.t[4];
    const uint32_t ta = c2 ? sb.t[6] : sb.t[2];
    const uint32_t c1 = ab > ta;
    const uint32_t th = c1 ? sb.t[7] : sb.t[5];
    const uint32_t tl = c1 ? sb.t[3] : sb.t[1];
    const uint32_t m2 = c2 + c2 + c1;
    m = m2 + m2 + (ab > (c2 ? th : tl));
  }
  if constexpr (BM == 0) return 0u;
  return m ^ (pos ? K2 : K2 - 1u);
}

template <int BM>
__device__ __forceinline__ float scaled_mag(const ScaledBook& sb, uint32_t m) {
  if constexpr (BM <= 1) return sb.c[0];
  float c = (m & 1) ? sb.c[1] : sb.c[0];
  if constexpr (BM >= 3) {
    const float c23 = (m & 1) ? sb.c[3] : sb.c[2];
    c = (m & 2) ? c23 : c;
  }
  if constexpr (BM >= 4) {
    const float c45 = (m & 1) ? sb.c[5] : sb.c[4];
    const float c67 = (m & 1) ? sb.c[7] : sb.c[6];
    const float chi = (m & 2) ? c67 : c45;
    c = (m & 4) ? chi : c;
  }
  return c;
}

template <int BM>
__device__ __forceinline__ float centroid_mag(const Book& bk, int m) {
  if constexpr (BM <= 1) return bk.c0;
  float c = (m & 1) ? bk.c1 : bk.c0;
  if constexpr (BM >= 3) {
    const float c23 = (m & 1) ? bk.c3 : bk.c2;
    c = (m & 2) ? c23 : c;
  }
  if constexpr (BM >= 4) {
    const float c45 = (m & 1) ? bk.c5 : bk.c4;
    const float c67 = (m & 1) ? bk.c7 : bk.c6;
    const float chi = (m & 2) ? c67 : c45;
    c = (m & 4) ? chi : c;
  }
  return c;
}

// Cell table of the nearest-centroid search (b_m >= 2). The code of y is
// idx = #{i : t_i < y} over the K - 1 signed thresholds t (the magnitudes
// tp[j] mirrored, t = 0 in the middle, as the search above reads them). On
// the accumulator acc = S·y (S > 0) the search compares acc with fl(t_i·S),
// exactly as the threshold search does. The cell of acc is the byte that
// f = acc·(128/S) + 128 converts to with saturation: whether the conversion
// floors or rounds, f lies in [k - 1/2, k + 1) for cell k, i.e. y in
// [(k - 128.5)/128, (k - 127)/128] up to rounding; cell 0 reaches down and
// cell 255 up without bound. Each cell is widened by 1/64 of its width on
// both sides and stores below = #{t_i below it} and the one threshold inside
// it (+inf if none), so idx = below + [acc > fl(t_inside·S)]. A codebook with
// two thresholds in one widened cell (spacing under ≈1.52/128) cannot use the
// table; the builder reports it and the encoder keeps the threshold search.
// PROD entries add the signed centroids of codes below and below + 1.
template <bool PROD>
using CellEntry = std::conditional_t<PROD, u32x4, u32x2>;

template <int BM, bool PROD>
__device__ __forceinline__ int build_cell(const Book& bk, int k, CellEntry<PROD>* cells) {
  constexpr int K = 1 << BM, H = K / 2;
  const float tp[8] = {0.f, bk.t1, bk.t2, bk.t3, bk.t4, bk.t5, bk.t6, bk.t7};
  const float cm[8] = {bk.c0, bk.c1, bk.c2, bk.c3, bk.c4, bk.c5, bk.c6, bk.c7};
  const float lo = k == 0 ? -INFINITY : (float(k) - 128.5f - 1.0f / 64) * (1.0f / 128);
  const float hi = k == 255 ? INFINITY : (float(k) - 127.0f + 1.0f / 64) * (1.0f / 128);
  int below = 0, inside = 0;
  float cand = INFINITY;
#pragma unroll
  for (int i = 0; i < K - 1; ++i) {
    const float t = i < H - 1 ? -tp[H - 1 - i] : tp[i - (H - 1)];
    if (t < lo) {
      ++below;
    } else if (t <= hi) {
      if (inside == 0) cand = t;
      ++inside;
    }
  }
  if constexpr (!PROD) {
    cells[k] = u32x2{uint32_t(below), __builtin_bit_cast(uint32_t, cand)};
  } else {
    float c0 = 0.f, c1 = 0.f;   // signed centroid of codes below and below + 1
#pragma unroll
    for (int c = 0; c < K; ++c) {
      const float v = c >= H ? cm[c - H] : -cm[H - 1 - c];
      c0 = c == below ? v : c0;
      c1 = c == below + 1 ? v : c1;
    }
    cells[k] = u32x4{uint32_t(below), __builtin_bit_cast(uint32_t, cand), __builtin_bit_cast(uint32_t, c0),
                     __builtin_bit_cast(uint32_t, c1)};
  }
  return inside > 1;
}

// Wavefronts per workgroup of the full-size encoder. Encodes with a cell
// table (b_m >= 2) run one workgroup per compute unit that shares one staged
// copy of the fragments: 16 wavefronts for mse (with a conflict-free table,
// below), 12 for prod (three per SIMD, as many as its registers allow). The
// other mse encodes run two workgroups of 8, the other prod encodes one.
template <int BM, bool PROD>
constexpr int enc_waves() { return BM >= 2 ? (PROD ? 12 : 16) : kEncWaves; }

template <int BM, bool PROD, bool F32IN>
__global__ __launch_bounds__((enc_waves<BM, PROD>() * 64)) void encode_kernel(EncodeArgs a) {
  constexpr int K = 1 << BM;
  constexpr bool kCells = BM >= 2;
  constexpr int kW = enc_waves<BM, PROD>();
  // mse: 32 interleaved copies of the cell table (entry k of copy c at
  // 256k + 8c bytes, c = lane % 32), so the 32 lanes of a half-wavefront read
  // 32 different bank pairs whatever their cells; prod (16-byte entries,
  // with S' staged too) keeps one copy. (Declared first: at LDS offset 0 the
  // lookups need no base address.)
  constexpr int kCellCopies = (kCells && !PROD) ? 32 : 1;
  __shared__ __attribute__((aligned(256))) CellEntry<PROD> lds_cells[kCells ? 256 * kCellCopies : 1];
  __shared__ u32x4 lds_rot[kFragsPerSet * 64];
  __shared__ u32x4 lds_proj[PROD ? kFragsPerSet * 64 : 1];
  const u32x4* frot = lds_rot;
  const u32x4* fproj = lds_proj;

  // Stage the operand fragments with direct-to-LDS loads (1 KiB per wavefront
  // instruction), all issued before a single wait.
  stage_frags(a.prep, lds_rot, PROD ? lds_proj : nullptr, threadIdx.x);
  const float rot_scale =
      reinterpret_cast<const PrepHeader*>(reinterpret_cast<const uint8_t*>(a.prep) - kPrepHeaderBytes)->rot_scale;
  Book bk{};
  if constexpr (BM >= 1) {
    const float* tb = a.boundaries + (K / 2 - 1);
    const float* cb = a.centroids + K / 2;
    bk.c0 = cb[0];
    if constexpr (K / 2 > 1) { bk.t1 = tb[1]; bk.c1 = cb[1]; }
    if constexpr (K / 2 > 2) { bk.t2 = tb[2]; bk.t3 = tb[3]; bk.c2 = cb[2]; bk.c3 = cb[3]; }
    if constexpr (K / 2 > 4) {
      bk.t4 = tb[4]; bk.t5 = tb[5]; bk.t6 = tb[6]; bk.t7 = tb[7];
      bk.c4 = cb[4]; bk.c5 = cb[5]; bk.c6 = cb[6]; bk.c7 = cb[7];
    }
  }
  int bad_cell = 0;
  if constexpr (kCells) {
    if (threadIdx.x < 256) bad_cell = build_cell<BM, PROD>(bk, threadIdx.x, lds_cells);
    if constexpr (kCellCopies > 1) {
      // entry k was built at index k; spread it to its copies at 32k + c
      // (every (k, c) read before any is written)
      constexpr int kPer = 256 * kCellCopies / (kW * 64);
      __syncthreads();
      CellEntry<PROD> e[kPer];
#pragma unroll
      for (int r = 0; r < kPer; ++r) e[r] = lds_cells[(threadIdx.x + kW * 64 * r) >> 5];
      __syncthreads();
#pragma unroll
      for (int r = 0; r < kPer; ++r) lds_cells[threadIdx.x + kW * 64 * r] = e[r];
    }
  }
  // A full barrier (with its memory fence) publishes the table; then the vote.
  __syncthreads();
  const bool use_cells = kCells && !__syncthreads_or(bad_cell);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const uint32_t cell_lane = 8u * uint32_t(lane & 31);   // the lane's table copy
  const int64_t ntiles = (a.n + 15) / 16;
  const int64_t tstride = int64_t(gridDim.x) * kW;
  // Raw input words of this lane's row for one tile: columns 32s + 8g + j.
  // The next tile's words are loaded while the current one is computed.
  constexpr int kRaw = F32IN ? 8 : 4;
  auto load_raw = [&](int64_t tile, u32x4 (&raw)[kRaw]) {
    const int64_t rowi = tile * 16 + n;
    const int64_t row = rowi < a.n ? rowi : a.n - 1;
    if constexpr (!F32IN) {
      const uint16_t* xr = static_cast<const uint16_t*>(a.x) + row * a.stride + 8 * g;
#pragma unroll
      for (int s = 0; s < 4; ++s) raw[s] = *reinterpret_cast<const u32x4*>(xr + 32 * s);
    } else {
      const float* xr = static_cast<const float*>(a.x) + row * a.stride + 8 * g;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        raw[2 * s] = *reinterpret_cast<const u32x4*>(xr + 32 * s);
        raw[2 * s + 1] = *reinterpret_cast<const u32x4*>(xr + 32 * s + 4);
      }
    }
  };
  // The tile loop, with the cell table (USE) or the threshold search.
  auto tiles = [&](auto use_tag) {
    constexpr bool USE = decltype(use_tag)::value;
    // (bf16 input only; fp32 input, twice the registers, loads its tile in place.)
    u32x4 raw_next[kRaw];
    int64_t tile = int64_t(blockIdx.x) * kW + wave;
    if (!F32IN && tile < ntiles) load_raw(tile, raw_next);
    for (; tile < ntiles; tile += tstride) {
      u32x4 raw[kRaw];
      if constexpr (F32IN) {
        load_raw(tile, raw);
      } else {
#pragma unroll
        for (int k = 0; k < kRaw; ++k) raw[k] = raw_next[k];
        if (tile + tstride < ntiles) load_raw(tile + tstride, raw_next);
      }
      const int64_t rowi = tile * 16 + n;
      const bool valid = rowi < a.n;
      const int64_t row = valid ? rowi : a.n - 1;
      const int64_t vec = a.slot ? a.slot[row] : row;   // output slot
      // The operand fragments in LDS are the same every tile; an opaque lane
      // offset keeps the compiler from hoisting all 64 KiB of them into
      // registers ahead of the loop.
      int lofs = lane;
      asm volatile("" : "+v"(lofs));

      // Columns held by this lane: slot 8s + j <-> column 32s + 8g + j. The
      // row is used as it is or scaled by 2^-e (row_exponent).
      float xv[32];
      if constexpr (!F32IN) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            xv[8 * s + 2 * k] = bf16_to_f32(raw[s][k] & 0xffffu);
            xv[8 * s + 2 * k + 1] = bf16_to_f32(raw[s][k] >> 16);
          }
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const f32x4 w0 = __builtin_bit_cast(f32x4, raw[2 * s]);
          const f32x4 w1 = __builtin_bit_cast(f32x4, raw[2 * s + 1]);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            xv[8 * s + k] = w0[k];
            xv[8 * s + 4 + k] = w1[k];
          }
        }
      }
      float ss = row_ss<F32IN>(xv);
      const int ex = row_exponent<F32IN>(xv, ss);
      const float rs = sqrtf(ss);                 // ‖x‖·2^-e
      const float nrm = ldexpf(rs, ex);
      u32x4 bx[4], bxl[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if constexpr (!F32IN) {
            bx[s][k] = bf16_row_pair(xv[8 * s + 2 * k], xv[8 * s + 2 * k + 1]);
          } else {
            uint16_t h0, l0, h1, l1;
            split_h(xv[8 * s + 2 * k], h0, l0);
            split_h(xv[8 * s + 2 * k + 1], h1, l1);
            bx[s][k] = uint32_t(h0) | (uint32_t(h1) << 16);
            bxl[s][k] = uint32_t(l0) | (uint32_t(l1) << 16);
          }
        }

      f32x4 acc[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const u32x4 ah = frot[frag_index(0, t, s) * 64 + lofs];
          const u32x4 al = frot[frag_index(1, t, s) * 64 + lofs];
          acc[t] = mfma(ah, bx[s], acc[t]);
          acc[t] = mfma(al, bx[s], acc[t]);
          if constexpr (F32IN) acc[t] = mfma(ah, bxl[s], acc[t]);
        }
      }

      // Row tile t, element j is rotated coordinate 32g + q, q = 4t + j, and
      // acc = S·y with S = 16‖x‖·2^-e (any S > 0 for a zero vector, whose acc is 0).
      const float S = (rs > 0.f) ? rot_scale * rs : 1.0f;
      // mse uses 1/S only for the cell lookup, whose cells are widened by far
      // more than the hardware reciprocal's error: one instruction instead of a
      // division. prod scales residuals and γ by it: the rounded quotient.
      const float up = PROD ? 1.0f / S : __builtin_amdgcn_rcpf(S);
      const float inv128 = 128.0f * up;
      ScaledBook sb;
      if constexpr (!USE) {
        const float tb[8] = {0.f, bk.t1, bk.t2, bk.t3, bk.t4, bk.t5, bk.t6, bk.t7};
        const float cb[8] = {bk.c0, bk.c1, bk.c2, bk.c3, bk.c4, bk.c5, bk.c6, bk.c7};
#pragma unroll
        for (int j = 1; j < K / 2; ++j) sb.t[j] = __builtin_bit_cast(uint32_t, tb[j] * S);
        if constexpr (PROD) {
#pragma unroll
          for (int j = 0; j < (K / 2 > 0 ? K / 2 : 1); ++j) sb.c[j] = cb[j] * S;
        }
      }
      uint32_t w[BM > 0 ? BM : 1];
#pragma unroll
      for (int k = 0; k < (BM > 0 ? BM : 1); ++k) w[k] = 0u;
      u32x4 brh[4], brl[4];
      float r2 = 0.f;
      const float rsc = up * kResScale;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        float res[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t m = 0u, code;
          bool pos = false;
          float cell_c = 0.f;      // USE: the signed centroid of the code
          if constexpr (USE) {
            // (Entry words are read as floats through __uint_as_float:
            // `__builtin_bit_cast` of a vector element in place compiled to a
            // read of element 0.)
            const float f = fmaf(acc[t][j], inv128, 128.0f);
            const uint32_t k = __builtin_amdgcn_cvt_pk_u8_f32(f, 0, 0u);
            if constexpr (PROD) {
              const u32x4 e = lds_cells[k];
              const bool up1 = acc[t][j] > __uint_as_float(e[1]) * S;
              code = e[0] + (up1 ? 1u : 0u);
              cell_c = __uint_as_float(up1 ? e[3] : e[2]);
            } else {
              // byte offset 256·cell + 8·(lane % 32): the conversion writes the
              // cell into byte 1 of the lane's copy offset
              const uint32_t off = __builtin_amdgcn_cvt_pk_u8_f32(f, 1, cell_lane);
              const u32x2 e = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(lds_cells) + off);
              code = e[0] + (acc[t][j] > __uint_as_float(e[1]) * S ? 1u : 0u);
            }
          } else {
            code = quantize_scaled<BM>(acc[t][j], sb, m, pos);
          }
          if constexpr (BM > 0) {
            const int q = 4 * t + j;
            const int bit = q * BM, wi = bit >> 5, off = bit & 31;
            w[wi] |= code << off;
            if (off + BM > 32) w[wi + 1] |= code >> (32 - off);
          }
          if constexpr (PROD) {
            float c = 0.f;
            if constexpr (USE) {
              c = cell_c * S;                      // = ±fl(|c|·S), as below
              asm volatile("" : "+v"(c));          // rounded product: no fused multiply-add
            } else if constexpr (BM >= 1) {
              c = scaled_mag<BM>(sb, m);
              c = pos ? c : -c;
            }
            const float racc = acc[t][j] - c;      // S·(y - c)
            r2 = fmaf(racc, racc, r2);
            res[j] = racc * rsc;                   // 64·(y - c)
          }
        }
        if constexpr (PROD) {
          // q = 4t + j  ->  K-step s = t/2, dword 2(t%2) + j/2, half j%2.
          uint16_t h0, l0, h1, l1, h2, l2, h3, l3;
          split_h(res[0], h0, l0);
          split_h(res[1], h1, l1);
          split_h(res[2], h2, l2);
          split_h(res[3], h3, l3);
          const int s = t >> 1, k0 = 2 * (t & 1);
          brh[s][k0] = uint32_t(h0) | (uint32_t(h1) << 16);
          brh[s][k0 + 1] = uint32_t(h2) | (uint32_t(h3) << 16);
          brl[s][k0] = uint32_t(l0) | (uint32_t(l1) << 16);
          brl[s][k0 + 1] = uint32_t(l2) | (uint32_t(l3) << 16);
        }
      }

      if constexpr (BM > 0) {
        if (valid) {
          uint32_t* dst = reinterpret_cast<uint32_t*>(a.codes + vec * (16 * BM) + 4 * BM * g);
          if constexpr (BM == 4) {
            *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
          } else if constexpr (BM == 2) {
            *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
          } else {
#pragma unroll
            for (int k = 0; k < BM; ++k) dst[k] = w[k];
          }
        }
      }
      if (valid && g == 0) a.norms[vec] = nrm;

      if constexpr (PROD) {
        r2 = sum4g(r2);
        f32x4 z[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) z[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const u32x4 sh = fproj[frag_index(0, t, s) * 64 + lofs];
            const u32x4 sl = fproj[frag_index(1, t, s) * 64 + lofs];
            z[t] = mfma(sh, brh[s], z[t]);
            z[t] = mfma(sl, brh[s], z[t]);
            z[t] = mfma(sh, brl[s], z[t]);
          }
        }
        uint32_t bits = 0u;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
#pragma unroll
          for (int j = 0; j < 4; ++j) bits |= uint32_t(z[t][j] >= 0.f) << (4 * t + j);
        }
        if (valid) {
          *reinterpret_cast<uint32_t*>(a.qjl + vec * 16 + 4 * g) = bits;
          if (g == 0) a.gammas[vec] = sqrtf(r2) * up;
        }
      }
    }
  };
  if (use_cells)
    tiles(std::integral_constant<bool, kCells>{});
  else
    tiles(std::integral_constant<bool, false>{});
}

// Encodes of at most this many 16-row tiles take the row-tile-parallel form:
// one workgroup per tile, no staging of the fragments in LDS.
constexpr int64_t kRowTileMax = 64;

__global__ __launch_bounds__(kRowWaves * 64) void row_encode_kernel(RowEncArgs a) {
  __shared__ RowXchg X;
  row_encode(a, blockIdx.x, X);
}

// Outlier-channel split encode ("TurboQuant của Google…" (omelet.tech),
// section "Thực nghiệm: 3.5 bit…"): two TurboQuant-mse instances in one pass.
// The block-structured Π puts the 32 outlier channels' rotation in the rows
// p mod 8 < 2 and the 96 regular channels' in the others, so one product
// rotates both groups; each group is then normalised by its own norm (from
// the input channels that the prepared mask marks) and quantized with its own
// codebook: BM + 1 bits on outlier rows, BM on the others. Lane (n, g) holds
// rotated coordinates 32g + q, q = 4t + j; q is an outlier position when
// t is even and j < 2. Its 32 codes form the bits [g·(32·BM + 8), (g+1)·(32·BM + 8))
// of the vector's code string (byte aligned), written byte by byte.
//
// PROD (prod keys): each group is a TurboQuant-prod instance. The residual of
// a coordinate is taken in its group's scale, S_g·(y - c), as in the unsplit
// encoder; the sketch runs on the block-structured S' = S·Πᵀ of the prepared
// buffer (zero across the groups), so one product gives both groups' sketch
// values at their positions; γ_o and γ_r are the groups' residual norms.
template <int BM, bool F32IN, bool PROD>
__global__ __launch_bounds__(kEncWaves * 64) void encode_split_kernel(EncodeArgs a) {
  constexpr int BO = BM + 1;
  constexpr int SEG = 32 * BM + 8;           // bits of a lane's 32 codes
  constexpr int NW = (SEG + 31) / 32;
  constexpr int ROW = 16 * BM + 4;           // bytes of a vector's codes
  __shared__ u32x4 lds_rot[kFragsPerSet * 64];
  __shared__ u32x4 lds_proj[PROD ? kFragsPerSet * 64 : 1];
  stage_frags(a.prep, lds_rot, PROD ? lds_proj : nullptr, threadIdx.x);
  const PrepHeader* hdr =
      reinterpret_cast<const PrepHeader*>(reinterpret_cast<const uint8_t*>(a.prep) - kPrepHeaderBytes);
  const float rot_scale = hdr->rot_scale;
  const Book br = load_book<BM>(a.centroids, a.boundaries);
  const Book bo = load_book<BO>(a.centroids_o, a.boundaries_o);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  // bit 8s + j: the lane's input column 32s + 8g + j is an outlier channel
  uint32_t omask = 0u;
#pragma unroll
  for (int s = 0; s < 4; ++s) omask |= ((hdr->omask[s] >> (8 * g)) & 0xffu) << (8 * s);
  // Cell tables of both groups' searches (as in encode_kernel; the regular
  // group's only at 3 bits): threads 0-255 build the outlier group's, 256-511
  // the regular group's.
  constexpr bool kCellsR = BM >= 3;
  __shared__ u32x2 cells_o[256];
  __shared__ u32x2 cells_r[kCellsR ? 256 : 1];
  int bad_cell = 0;
  if (threadIdx.x < 256)
    bad_cell = build_cell<BO, false>(bo, threadIdx.x, cells_o);
  else if (kCellsR)
    bad_cell = build_cell<(kCellsR ? BM : 3), false>(br, threadIdx.x - 256, cells_r);
  __syncthreads();
  const bool use_cells = !__syncthreads_or(bad_cell);

  const int64_t ntiles = (a.n + 15) / 16;
  const int64_t tstride = int64_t(gridDim.x) * kEncWaves;
  // The tile loop, with the cell tables (USE) or the threshold searches.
  auto tiles = [&](auto use_tag) {
    constexpr bool USE = decltype(use_tag)::value;
    for (int64_t tile = int64_t(blockIdx.x) * kEncWaves + wave; tile < ntiles; tile += tstride) {
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
      int lofs = lane;
      asm volatile("" : "+v"(lofs));
      float xv[32];
      if constexpr (!F32IN) {
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
      // the row as it is or scaled by 2^-e, as in the unsplit encoder
      float ss = row_ss<F32IN>(xv);
      const int ex = row_exponent<F32IN>(xv, ss);
      float sso = 0.f, ssr = 0.f;
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        const float v2 = xv[q] * xv[q];
        if ((omask >> q) & 1u)
          sso += v2;
        else
          ssr += v2;
      }
      sso = sum4g(sso);
      ssr = sum4g(ssr);
      const float rso = sqrtf(sso), rsr = sqrtf(ssr);
      u32x4 bx[4], bxl[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if constexpr (!F32IN) {
            bx[s][k] = bf16_row_pair(xv[8 * s + 2 * k], xv[8 * s + 2 * k + 1]);
          } else {
            uint16_t h0, l0, h1, l1;
            split_h(xv[8 * s + 2 * k], h0, l0);
            split_h(xv[8 * s + 2 * k + 1], h1, l1);
            bx[s][k] = uint32_t(h0) | (uint32_t(h1) << 16);
            bxl[s][k] = uint32_t(l0) | (uint32_t(l1) << 16);
          }
        }
      f32x4 acc[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const u32x4 ah = lds_rot[frag_index(0, t, s) * 64 + lofs];
          const u32x4 al = lds_rot[frag_index(1, t, s) * 64 + lofs];
          acc[t] = mfma(ah, bx[s], acc[t]);
          acc[t] = mfma(al, bx[s], acc[t]);
          if constexpr (F32IN) acc[t] = mfma(ah, bxl[s], acc[t]);
        }
      }
      // acc = rot_scale·Π·x·2^-e; a group's rotated unit vector is its rows
      // over rot_scale·‖x_g‖·2^-e, so the thresholds scale by that
      const float So = rso > 0.f ? rot_scale * rso : 1.0f;
      const float Sr = rsr > 0.f ? rot_scale * rsr : 1.0f;
      ScaledBook sbo, sbr;
      const float inv_o = 128.0f / So, inv_r = 128.0f / Sr;
      // Scaled thresholds of the groups that search without a cell table.
      if constexpr (!USE) {
        const float to[8] = {0.f, bo.t1, bo.t2, bo.t3, bo.t4, bo.t5, bo.t6, bo.t7};
#pragma unroll
        for (int j = 1; j < (1 << BO) / 2; ++j) sbo.t[j] = __builtin_bit_cast(uint32_t, to[j] * So);
      }
      if constexpr (!USE || !kCellsR) {
        const float tr[8] = {0.f, br.t1, br.t2, br.t3, br.t4, br.t5, br.t6, br.t7};
#pragma unroll
        for (int j = 1; j < (1 << BM) / 2; ++j) sbr.t[j] = __builtin_bit_cast(uint32_t, tr[j] * Sr);
      }
      if constexpr (PROD) {
        // the groups' centroid magnitudes in their scales, fl(|c|·S_g)
        const float co[8] = {bo.c0, bo.c1, bo.c2, bo.c3, bo.c4, bo.c5, bo.c6, bo.c7};
        const float cr[8] = {br.c0, br.c1, br.c2, br.c3, br.c4, br.c5, br.c6, br.c7};
#pragma unroll
        for (int j = 0; j < (1 << BO) / 2; ++j) sbo.c[j] = co[j] * So;
#pragma unroll
        for (int j = 0; j < ((1 << BM) / 2 > 0 ? (1 << BM) / 2 : 1); ++j) sbr.c[j] = cr[j] * Sr;
      }
      uint32_t w[NW];
#pragma unroll
      for (int k = 0; k < NW; ++k) w[k] = 0u;
      u32x4 brh[4], brl[4];
      float r2o = 0.f, r2r = 0.f;
      const float rsco = kResScale / So, rscr = kResScale / Sr;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        float res[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int q = 4 * t + j, c = q >> 3, r = q & 7;
          const bool out = r < 2;
          uint32_t m = 0u;
          bool pos = false;
          uint32_t code;
          if (USE && (out || kCellsR)) {
            // cell of acc in the group's table: idx = below + [acc > fl(t·S)]
            const float Sg = out ? So : Sr;
            const float f = fmaf(acc[t][j], out ? inv_o : inv_r, 128.0f);
            const uint32_t k = __builtin_amdgcn_cvt_pk_u8_f32(f, 0, 0u);
            const u32x2 e = out ? cells_o[k] : cells_r[kCellsR ? k : 0];
            code = e[0] + (acc[t][j] > __uint_as_float(e[1]) * Sg ? 1u : 0u);
            if constexpr (PROD) {
              // the code's magnitude index and sign
              const uint32_t h = out ? (1u << BO) / 2 : (1u << BM) / 2;
              pos = code >= h;
              m = pos ? code - h : h - 1u - code;
            }
          } else {
            code = out ? quantize_scaled<BO>(acc[t][j], sbo, m, pos) : quantize_scaled<BM>(acc[t][j], sbr, m, pos);
          }
          const int width = out ? BO : BM;
          const int bit = c * (8 * BM + 2) + (out ? r * BO : 2 * BO + (r - 2) * BM);
          const int wi = bit >> 5, off = bit & 31;
          w[wi] |= code << off;
          if (off + width > 32) w[wi + 1] |= code >> (32 - off);
          if constexpr (PROD) {
            float cv = out ? scaled_mag<BO>(sbo, m) : scaled_mag<BM>(sbr, m);
            cv = pos ? cv : -cv;
            const float racc = acc[t][j] - cv;                 // S_g·(y - c)
            if (out)
              r2o = fmaf(racc, racc, r2o);
            else
              r2r = fmaf(racc, racc, r2r);
            res[j] = racc * (out ? rsco : rscr);               // 64·(y - c)
          }
        }
        if constexpr (PROD) {
          // q = 4t + j  ->  K-step s = t/2, dword 2(t%2) + j/2, half j%2.
          uint16_t h0, l0, h1, l1, h2, l2, h3, l3;
          split_h(res[0], h0, l0);
          split_h(res[1], h1, l1);
          split_h(res[2], h2, l2);
          split_h(res[3], h3, l3);
          const int s = t >> 1, k0 = 2 * (t & 1);
          brh[s][k0] = uint32_t(h0) | (uint32_t(h1) << 16);
          brh[s][k0 + 1] = uint32_t(h2) | (uint32_t(h3) << 16);
          brl[s][k0] = uint32_t(l0) | (uint32_t(l1) << 16);
          brl[s][k0 + 1] = uint32_t(l2) | (uint32_t(l3) << 16);
        }
      }
      if (valid) {
        uint8_t* dst = a.codes + vec * ROW + g * (SEG / 8);
#pragma unroll
        for (int k = 0; k < SEG / 8; ++k) dst[k] = static_cast<uint8_t>(w[k >> 2] >> (8 * (k & 3)));
        if (g == 0) {
          a.norms[2 * vec] = ldexpf(rso, ex);
          a.norms[2 * vec + 1] = ldexpf(rsr, ex);
        }
      }
      if constexpr (PROD) {
        r2o = sum4g(r2o);
        r2r = sum4g(r2r);
        f32x4 z[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) z[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const u32x4 sh = lds_proj[frag_index(0, t, s) * 64 + lofs];
            const u32x4 sl = lds_proj[frag_index(1, t, s) * 64 + lofs];
            z[t] = mfma(sh, brh[s], z[t]);
            z[t] = mfma(sl, brh[s], z[t]);
            z[t] = mfma(sh, brl[s], z[t]);
          }
        }
        uint32_t bits = 0u;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
#pragma unroll
          for (int j = 0; j < 4; ++j) bits |= uint32_t(z[t][j] >= 0.f) << (4 * t + j);
        }
        if (valid) {
          *reinterpret_cast<uint32_t*>(a.qjl + vec * 16 + 4 * g) = bits;
          if (g == 0) {
            a.gammas[2 * vec] = sqrtf(r2o) / So;
            a.gammas[2 * vec + 1] = sqrtf(r2r) / Sr;
          }
        }
      }
    }
  };
  if (use_cells)
    tiles(std::integral_constant<bool, true>{});
  else
    tiles(std::integral_constant<bool, false>{});
}

template <int BM, bool PROD>
hipError_t launch_encode_t(const EncodeArgs& a, bool f32in, int grid, hipStream_t st) {
  if (f32in)
    hipLaunchKernelGGL((encode_kernel<BM, PROD, true>), dim3(grid), dim3(enc_waves<BM, PROD>() * 64), 0, st, a);
  else
    hipLaunchKernelGGL((encode_kernel<BM, PROD, false>), dim3(grid), dim3(enc_waves<BM, PROD>() * 64), 0, st, a);
  return hipGetLastError();
}

}  // namespace tq

using namespace tq;

namespace {
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_quantizer(const tq_quantizer* q) {
  if (q == nullptr) return TQ_ERR_INVALID_ARG;
  if (q->d != TQ_HEAD_DIM) return TQ_ERR_UNSUPPORTED;
  if (q->variant != TQ_MSE && q->variant != TQ_PROD) return TQ_ERR_UNSUPPORTED;
  if (q->bits < 1 || q->bits > 4) return TQ_ERR_UNSUPPORTED;
  const int bm = q->variant == TQ_PROD ? q->bits - 1 : q->bits;
  if (q->centroids == nullptr || q->prep == nullptr) return TQ_ERR_INVALID_ARG;
  if (q->split == TQ_SPLIT_NONE && q->rot == nullptr) return TQ_ERR_INVALID_ARG;
  if (bm > 0 && q->boundaries == nullptr) return TQ_ERR_INVALID_ARG;
  if (q->variant == TQ_PROD && q->split == TQ_SPLIT_NONE && q->proj == nullptr) return TQ_ERR_INVALID_ARG;
  if (!aligned(q->prep, 256)) return TQ_ERR_WORKSPACE;
  if (q->rotation != TQ_ROT_DENSE && q->rotation != TQ_ROT_HADAMARD) return TQ_ERR_UNSUPPORTED;
  if (q->split != TQ_SPLIT_NONE && q->split != TQ_SPLIT_OUTLIER32) return TQ_ERR_UNSUPPORTED;
  if (q->split == TQ_SPLIT_OUTLIER32) {
    if (q->bits < 2 || q->bits > 3 || q->rotation != TQ_ROT_DENSE) return TQ_ERR_UNSUPPORTED;
    if (q->centroids_o == nullptr || q->boundaries_o == nullptr) return TQ_ERR_INVALID_ARG;
    if (q->rot_o == nullptr || q->rot_r == nullptr || q->channels_o == nullptr) return TQ_ERR_INVALID_ARG;
    if (q->variant == TQ_PROD && (q->proj_o == nullptr || q->proj_r == nullptr)) return TQ_ERR_INVALID_ARG;
  }
  return TQ_OK;
}

// The caller's outlier channels: 32 distinct values in [0, d).
bool channels_valid(const int32_t* ch) {
  uint32_t seen[4] = {0u, 0u, 0u, 0u};
  for (int j = 0; j < 32; ++j) {
    const int32_t c = ch[j];
    if (c < 0 || c >= TQ_HEAD_DIM || ((seen[c >> 5] >> (c & 31)) & 1u)) return false;
    seen[c >> 5] |= 1u << (c & 31);
  }
  return true;
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return cus;
}
}  // namespace

extern "C" size_t tq_prep_bytes(void) { return kPrepBytes; }

namespace {
template <int BM, bool PROD>
void launch_split_t(const EncodeArgs& a, bool f32, dim3 grid, hipStream_t s) {
  if (f32)
    hipLaunchKernelGGL((encode_split_kernel<BM, true, PROD>), grid, dim3(kEncWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL((encode_split_kernel<BM, false, PROD>), grid, dim3(kEncWaves * 64), 0, s, a);
}

int launch_split(const tq_quantizer* q, const EncodeArgs& a, bool f32, hipStream_t s) {
  const bool prod = q->variant == TQ_PROD;
  const int64_t tiles = (a.n + 15) / 16;
  const int64_t want = (tiles + kEncWaves - 1) / kEncWaves;
  const int cap = device_cus() * (prod ? 1 : 2);
  const dim3 grid(static_cast<unsigned>(want < cap ? want : cap));
  if (!prod) {
    if (q->bits == 2)
      launch_split_t<2, false>(a, f32, grid, s);
    else
      launch_split_t<3, false>(a, f32, grid, s);
  } else {
    if (q->bits == 2)
      launch_split_t<1, true>(a, f32, grid, s);
    else
      launch_split_t<2, true>(a, f32, grid, s);
  }
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}
}  // namespace

extern "C" int tq_prepare(const tq_quantizer* q, void* stream) {
  const int st = check_quantizer(q);
  if (st != TQ_OK) return st;
  const int bm = q->variant == TQ_PROD ? q->bits - 1 : q->bits;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float* rot = q->rot;
  const float* proj = q->proj;
  if (q->split == TQ_SPLIT_OUTLIER32) {
    // the whole rotation as one block-structured matrix, built in the
    // prepared buffer from the caller's Π_o, Π_r and outlier channels
    if (!channels_valid(q->channels_o)) return TQ_ERR_INVALID_ARG;
    SplitChannels ch;
    for (int c = 0; c < TQ_HEAD_DIM; ++c) ch.slot[c] = -1;
    for (int j = 0; j < 32; ++j) ch.slot[q->channels_o[j]] = j;
    int r = 32;
    for (int c = 0; c < TQ_HEAD_DIM; ++c)
      if (ch.slot[c] < 0) ch.slot[c] = r++;
    float* block = reinterpret_cast<float*>(static_cast<uint8_t*>(q->prep) + kPrepRotOff);
    hipLaunchKernelGGL(split_rotation_kernel, dim3(kD), dim3(kD), 0, s, q->rot_o, q->rot_r, ch, block);
    if (hipGetLastError() != hipSuccess) return TQ_ERR_HIP;
    rot = block;
    if (q->variant == TQ_PROD) {
      // the sketch matrices in the same block structure (rows: sketch
      // positions; columns: channels)
      float* sblock = reinterpret_cast<float*>(static_cast<uint8_t*>(q->prep) + kPrepProjOff);
      hipLaunchKernelGGL(split_rotation_kernel, dim3(kD), dim3(kD), 0, s, q->proj_o, q->proj_r, ch, sblock);
      if (hipGetLastError() != hipSuccess) return TQ_ERR_HIP;
      proj = sblock;
    }
  }
  hipLaunchKernelGGL(prepare_kernel, dim3(1), dim3(1024), 0, s, rot, q->variant == TQ_PROD ? proj : nullptr,
                     q->centroids, bm,
                     q->rotation == TQ_ROT_HADAMARD ? 1 : 0,
                     q->split == TQ_SPLIT_OUTLIER32 ? q->centroids_o : nullptr, static_cast<uint8_t*>(q->prep));
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

extern "C" int tq_encode_chunked(const tq_quantizer* q, const void* x, int x_dtype, int64_t n, int chunks,
                                 int64_t x_row_stride, const tq_packed* out, void* stream) {
  int st = check_quantizer(q);
  if (st != TQ_OK) return st;
  if (chunks < 1 || n < 0 || out == nullptr) return TQ_ERR_INVALID_ARG;
  if (chunks > 64) return TQ_ERR_UNSUPPORTED;
  if (q->split != TQ_SPLIT_NONE) return TQ_ERR_UNSUPPORTED;
  if (x_row_stride < int64_t(chunks) * TQ_HEAD_DIM) return TQ_ERR_INVALID_ARG;
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return TQ_ERR_UNSUPPORTED;
  const size_t esz = x_dtype == TQ_F32 ? 4 : 2;
  const bool prod = q->variant == TQ_PROD;
  const int bm = prod ? q->bits - 1 : q->bits;
  const size_t code_row = size_t(TQ_HEAD_DIM) * bm / 8;
  // chunk c: the rows' coordinates 128c..128c+127, stored in slots c·n + i
  for (int c = 0; c < chunks; ++c) {
    const size_t row0 = size_t(c) * size_t(n);
    tq_packed o;
    o.codes = bm > 0 && out->codes != nullptr ? out->codes + row0 * code_row : nullptr;
    o.norms = out->norms != nullptr ? out->norms + row0 : nullptr;
    o.qjl = prod && out->qjl != nullptr ? out->qjl + row0 * (TQ_HEAD_DIM / 8) : nullptr;
    o.gammas = prod && out->gammas != nullptr ? out->gammas + row0 : nullptr;
    const void* xc = x != nullptr ? static_cast<const uint8_t*>(x) + size_t(c) * TQ_HEAD_DIM * esz : nullptr;
    st = tq_encode(q, xc, x_dtype, n, x_row_stride, &o, nullptr, stream);
    if (st != TQ_OK) return st;
  }
  return TQ_OK;
}

// The decode step's append for split quantizers: rows r = b·hkv + h of x
// (already checked by the caller) into slot r·max_ctx + lens[b] - 1 of cache.
int tq_split_append(const tq_quantizer* q, const void* x, int x_dtype, int64_t rows, int64_t x_row_stride,
                    const tq_packed* cache, const int32_t* lens, int64_t max_ctx, int hkv, void* stream) {
  EncodeArgs a{};
  a.x = x;
  a.n = rows;
  a.stride = x_row_stride;
  a.codes = cache->codes;
  a.norms = cache->norms;
  a.qjl = cache->qjl;
  a.gammas = cache->gammas;
  a.prep = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(q->prep) + kPrepHeaderBytes);
  a.centroids = q->centroids;
  a.boundaries = q->boundaries;
  a.centroids_o = q->centroids_o;
  a.boundaries_o = q->boundaries_o;
  a.lens = lens;
  a.max_ctx = max_ctx;
  a.hkv = hkv;
  a.append = 1;
  return launch_split(q, a, x_dtype == TQ_F32, static_cast<hipStream_t>(stream));
}

// Exported for the decoder, which checks quantizers the same way.
int tq_check_quantizer(const tq_quantizer* q) { return check_quantizer(q); }
// The quantizer's whole d×d rotation as the decoder reads it (a split
// quantizer's is the block matrix in its prepared buffer).
const float* tq_rotation_matrix(const tq_quantizer* q) {
  return q->split == TQ_SPLIT_OUTLIER32
             ? reinterpret_cast<const float*>(static_cast<const uint8_t*>(q->prep) + kPrepRotOff)
             : q->rot;
}
// The same for the sketch matrix S of a prod quantizer (null for mse).
const float* tq_projection_matrix(const tq_quantizer* q) {
  if (q->variant != TQ_PROD) return nullptr;
  return q->split == TQ_SPLIT_OUTLIER32
             ? reinterpret_cast<const float*>(static_cast<const uint8_t*>(q->prep) + kPrepProjOff)
             : q->proj;
}
int tq_device_cus() { return device_cus(); }

extern "C" int tq_encode(const tq_quantizer* q, const void* x, int x_dtype, int64_t n,
                         int64_t x_row_stride, const tq_packed* out, const int64_t* out_slot,
                         void* stream) {
  int st = check_quantizer(q);
  if (st != TQ_OK) return st;
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return TQ_ERR_UNSUPPORTED;
  if (n < 0 || out == nullptr) return TQ_ERR_INVALID_ARG;
  if (n == 0) return TQ_OK;
  if (x == nullptr || x_row_stride < TQ_HEAD_DIM || (x_row_stride % 8) != 0) return TQ_ERR_INVALID_ARG;
  const bool prod = q->variant == TQ_PROD;
  const int bm = prod ? q->bits - 1 : q->bits;
  if (out->norms == nullptr || (bm > 0 && out->codes == nullptr)) return TQ_ERR_INVALID_ARG;
  if (prod && (out->qjl == nullptr || out->gammas == nullptr)) return TQ_ERR_INVALID_ARG;
  if (!aligned(x, 16) || (bm > 0 && !aligned(out->codes, 16)) || !aligned(out->norms, 4) ||
      (prod && (!aligned(out->qjl, 16) || !aligned(out->gammas, 4))))
    return TQ_ERR_INVALID_ARG;

  EncodeArgs a{};
  a.x = x;
  a.n = n;
  a.stride = x_row_stride;
  a.codes = out->codes;
  a.norms = out->norms;
  a.qjl = out->qjl;
  a.gammas = out->gammas;
  a.prep = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(q->prep) + kPrepHeaderBytes);
  a.centroids = q->centroids;
  a.boundaries = q->boundaries;
  a.slot = out_slot;
  a.centroids_o = q->centroids_o;
  a.boundaries_o = q->boundaries_o;
  const int64_t tiles = (n + 15) / 16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (q->split == TQ_SPLIT_OUTLIER32) return launch_split(q, a, x_dtype == TQ_F32, s);
  if (tiles <= kRowTileMax) {
    RowEncArgs r{};
    r.x = x;
    r.n = n;
    r.stride = x_row_stride;
    r.f32in = x_dtype == TQ_F32;
    r.bm = bm;
    r.prod = prod;
    r.codes = out->codes;
    r.norms = out->norms;
    r.qjl = out->qjl;
    r.gammas = out->gammas;
    r.frags = a.prep;
    r.centroids = q->centroids;
    r.boundaries = q->boundaries;
    r.slot = out_slot;
    hipLaunchKernelGGL(row_encode_kernel, dim3(static_cast<unsigned>(tiles)), dim3(kRowWaves * 64), 0, s, r);
    return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
  }
  // one workgroup per compute unit of 16 wavefronts for mse with a cell
  // table and of 12 for prod with one, two of 8 for the other mse encodes,
  // one of 8 for the other prod encodes
  const int waves = bm >= 2 ? (prod ? 12 : 16) : kEncWaves;
  const int64_t want = (tiles + waves - 1) / waves;
  const int cap = device_cus() * ((prod || bm >= 2) ? 1 : 2);
  const int grid = static_cast<int>(want < cap ? want : cap);
  const bool f32 = x_dtype == TQ_F32;
  hipError_t e;
  if (!prod) {
    switch (bm) {
      case 1: e = launch_encode_t<1, false>(a, f32, grid, s); break;
      case 2: e = launch_encode_t<2, false>(a, f32, grid, s); break;
      case 3: e = launch_encode_t<3, false>(a, f32, grid, s); break;
      default: e = launch_encode_t<4, false>(a, f32, grid, s); break;
    }
  } else {
    switch (bm) {
      case 0: e = launch_encode_t<0, true>(a, f32, grid, s); break;
      case 1: e = launch_encode_t<1, true>(a, f32, grid, s); break;
      case 2: e = launch_encode_t<2, true>(a, f32, grid, s); break;
      default: e = launch_encode_t<3, true>(a, f32, grid, s); break;
    }
  }
  return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

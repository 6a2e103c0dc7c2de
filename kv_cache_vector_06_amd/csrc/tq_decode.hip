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
//      group of <= 8 query heads). A workgroup of 8 wavefronts fills one
//      compute unit; each wavefront streams 32-token blocks through its LDS
//      ring: codes → fp16 operands through LDS lookup tables, scores on the
//      matrix cores (heads padded to 16 columns), online softmax reduced per
//      wavefront, P·V on the matrix cores into a rotated-space accumulator.
//      The wavefronts merge in LDS and write one partial (max, sum, acc[128])
//      per head.
//   3. merge: log-sum-exp combine of the splits, then o = Π_Vᵀ acc / sum.
//
// Precision (rel. L2 vs an fp64 evaluation ~1e-5..1e-4 on Llama-shaped data):
// centroids enter the fp16 tables as c·64·σ with a per-codebook σ in [1, 2)
// chosen by tq_prepare so that they are nearly fp16-exact (≤ 2e-5 relative
// error for ≤ 3-bit codebooks, ≤ 1e-4 for 4-bit ones, whose key table also
// carries the fp16 remainder); q' and q_S are split into fp16 hi + lo (held in
// separate matrix columns of one pass); the softmax weights are split hi + lo
// (separate matrix rows of one pass); all sums are fp32.
#include <hip/hip_runtime.h>
#include <math.h>

#include <mutex>

#include "tq.h"
#include "tq_device.h"
#include "tq_rowtile.h"

int tq_check_quantizer(const tq_quantizer* q);
const float* tq_rotation_matrix(const tq_quantizer* q);
const float* tq_projection_matrix(const tq_quantizer* q);
int tq_split_append(const tq_quantizer* q, const void* x, int x_dtype, int64_t rows, int64_t x_row_stride,
                    const tq_packed* cache, const int32_t* lens, int64_t max_ctx, int hkv, void* stream);

#define TQ_LDS(p) ((__attribute__((address_space(3))) void*)(p))

namespace tq {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kDecWaves = 8;             // wavefronts per split workgroup (2 per SIMD)
constexpr int kBlockTok = 32;            // tokens per wavefront step
constexpr int kMaxHeads = 8;             // query heads per unit
constexpr int kPartStride = 132;         // floats per (unit, split, head) partial: M, L, pad, pad, acc[128]
constexpr int kQFrags = 4;              // q' (hi | lo columns) × 4 K-steps
// Per unit: the fp16 fragments, the per-head score scales, then the sketch
// operand of the scaled fp4 × fp8 sketch products (split and search kernels; two
// products: 64 lanes × 32 fp8 bytes each) and their per-lane E8M0 scales.
constexpr size_t kSkOff = kQFrags * 1024 + 256;
constexpr size_t kSkScaleOff = kSkOff + 2 * 64 * 32;
constexpr size_t kUnitBytes = kSkScaleOff + 2 * 64 * 4;
constexpr int kTargetGroups = 256;       // split workgroups per launch: one per compute unit
constexpr int64_t kMaxSplitsPlan = 4096;        // splits per unit (merge keeps one weight each)
constexpr int64_t kMaxCtx = int64_t(1) << 26;   // tokens per (batch, KV head): 32-bit offsets

struct Plan {
  int ngroups, units, nsplit, split_len;
  size_t part_off, bytes;
};

inline Plan make_plan(int B, int Hq, int Hkv, int64_t max_ctx) {
  Plan p{};
  const int G = Hq / Hkv;
  p.ngroups = (G + kMaxHeads - 1) / kMaxHeads;
  p.units = B * Hkv * p.ngroups;
  // With fewer units than compute units, split the tokens so that one round
  // of workgroups covers the chip, keeping at least 8 blocks per wavefront.
  const int64_t gran = int64_t(kDecWaves) * kBlockTok;
  int64_t want = p.units >= kTargetGroups ? 1 : kTargetGroups / p.units;
  const int64_t max_by_len = (max_ctx + 8 * gran - 1) / (8 * gran);
  if (want > max_by_len) want = max_by_len;
  if (want < 1) want = 1;
  if (want > kMaxSplitsPlan) want = kMaxSplitsPlan;
  const int64_t per = (max_ctx + want - 1) / want;
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
  int Hq, Hkv, G, ngroups, units;
  uint8_t* ws;
  int64_t qstride = kD;   // floats between query rows (row b·Hq + head)
};

__device__ __forceinline__ int max_exponent(float (&v)[32]) {
  float m = 0.f;
#pragma unroll
  for (int q = 0; q < 32; ++q) m = fmaxf(m, fabsf(v[q]));
  m = max4g(m);
  int ex = 0;
  if (m > 0.f) frexpf(m, &ex);
  return ex;
}

__device__ __forceinline__ void split_pairs(const float (&v)[32], u32x4 (&hi)[4], u32x4 (&lo)[4]) {
  // v[q], q = 8s + 2k + h  ->  K-step s, dword k, half h
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint16_t h0, l0, h1, l1;
      split_h(v[8 * s + 2 * k], h0, l0);
      split_h(v[8 * s + 2 * k + 1], h1, l1);
      hi[s][k] = uint32_t(h0) | (uint32_t(h1) << 16);
      lo[s][k] = uint32_t(l0) | (uint32_t(l1) << 16);
    }
}

// OCP fp8 E4M3 (bias 7) of a finite y with |y| < 448, rounded to nearest
// even, and the value of a code. Prep-time only.
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
  const uint32_t sgn = y < 0.f ? 0x80u : 0u;
  const float a = fabsf(y);
  if (a < 0x1p-6f) return sgn | static_cast<uint32_t>(rintf(a * 512.0f));   // subnormals: units of 2^-9
  int e;
  const float m = frexpf(a, &e);                                             // a = 2m·2^(e-1), 2m in [1, 2)
  uint32_t q = static_cast<uint32_t>(rintf((2.0f * m - 1.0f) * 8.0f));
  int ex = e - 1;
  if (q == 8u) {
    q = 0u;
    ++ex;
  }
  return sgn | (static_cast<uint32_t>(ex + 7) << 3) | q;
}
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t ef = (c >> 3) & 15u, mf = c & 7u;
  const float mag = ef ? ldexpf(1.0f + 0.125f * static_cast<float>(mf), static_cast<int>(ef) - 7)
                       : 0x1p-9f * static_cast<float>(mf);
  return (c & 0x80u) ? -mag : mag;
}

// Four values of one column into the two dwords of fp16 pairs (v0, v1),
// (v2, v3) after scaling by scl: the hi parts, or the lo parts.
__device__ __forceinline__ u32x2 hilo_pairs(const float (&v)[4], float scl, bool hi) {
  uint16_t h[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) split_h(v[j] * scl, h[j], l[j]);
  return hi ? u32x2{uint32_t(h[0]) | (uint32_t(h[1]) << 16), uint32_t(h[2]) | (uint32_t(h[3]) << 16)}
            : u32x2{uint32_t(l[0]) | (uint32_t(l[1]) << 16), uint32_t(l[2]) | (uint32_t(l[3]) << 16)};
}

// Query operands of one unit, row-tile parallel: a workgroup of 8 wavefronts
// per unit, wavefront t forming rotated dims 32g + 4t + j (j < 4) of every
// column. q' = Π_K q and q_S = S q = S'·q' (S' = S·Πᵀ) run on the matrix cores
// with the key quantizer's prepared fragments, each in three hi/lo passes
// (fp16 hi/lo of the matrix times fp16 hi/lo of the power-of-two-scaled
// vector, fp32 sums), so both are fp32-accurate. The column maxima and the
// sketch's B operand meet in LDS. Columns n and n + 8 carry head n % 8: hi
// parts in n < 8, lo parts in n >= 8, so one pass of the split kernel's
// matrix cores gives both.
__device__ __forceinline__ void row_prep(const PrepArgs& a, int unit, RowXchg& X) {
  const int lane = threadIdx.x & 63;
  const int t = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int grp = unit % a.ngroups;
  const int kvh = (unit / a.ngroups) % a.Hkv;
  const int b = unit / (a.ngroups * a.Hkv);
  const int gc = min(kMaxHeads, a.G - grp * kMaxHeads);
  const int n = lane & 15, g = lane >> 4, c = n & 7;
  const bool live = c < gc;
  const bool prod = a.proj != nullptr;
  const u32x4* frag = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(a.kh) + kPrepHeaderBytes);
  // the header's scales, read up front (not after the products)
  const float rot_scale = scalar_load(&a.kh->rot_scale), sigma = scalar_load(&a.kh->sigma);
  const float sp_scale = prod ? scalar_load(&a.kh->sp_scale) : 1.0f;
  u32x4 rh[4], rl[4], ph[4], pl[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    rh[s] = frag[frag_index(0, t, s) * 64 + lane];
    rl[s] = frag[frag_index(1, t, s) * 64 + lane];
  }
  if (prod) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      ph[s] = frag[(kFragsPerSet + frag_index(0, t, s)) * 64 + lane];
      pl[s] = frag[(kFragsPerSet + frag_index(1, t, s)) * 64 + lane];
    }
  }
  // B operand of the rotation: slot 8s + j of this lane is dim 32s + 8g + j.
  float xv[32];
  {
    const float* qr =
        a.query + (size_t(b) * a.Hq + kvh * a.G + grp * kMaxHeads + (live ? c : 0)) * size_t(a.qstride) + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(qr + 32 * s);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(qr + 32 * s + 4);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        xv[8 * s + k] = live ? w0[k] : 0.f;
        xv[8 * s + 4 + k] = live ? w1[k] : 0.f;
      }
    }
  }
  const int ex = max_exponent(xv);
#pragma unroll
  for (int q = 0; q < 32; ++q) xv[q] = ldexpf(xv[q], -ex);
  u32x4 bh[4], bl[4];
  split_pairs(xv, bh, bl);
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    acc = mfma(rh[s], bh[s], acc);
    acc = mfma(rl[s], bh[s], acc);
    acc = mfma(rh[s], bl[s], acc);
  }
  float qp[4], qs[4];                            // dims 32g + 4t + j
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    qp[j] = ldexpf(acc[j], ex) / rot_scale;
    qs[j] = 0.f;
  }
  if (prod) {
    // B operand of the sketch: q' scaled by 2^-e2 (max|q'| = m·2^e2), split
    // hi/lo; K-step s, dword k of lane group g is dims 32g + 8s + 2k, +1.
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) m = fmaxf(m, fabsf(qp[j]));
    m = max4g(m);
    if (g == 0) X.red[0][t][n] = m;
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) m = fmaxf(m, X.red[0][tt][n]);
    int e2 = 0;
    if (m > 0.f) frexpf(m, &e2);
    float y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = ldexpf(qp[j], -e2);
    X.b[0][t][lane] = hilo_pairs(y, 1.0f, true);
    X.b[1][t][lane] = hilo_pairs(y, 1.0f, false);
    __syncthreads();
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
    const float inv = 1.0f / sp_scale;
#pragma unroll
    for (int j = 0; j < 4; ++j) qs[j] = ldexpf(z[j], e2) * inv;
  }
  // score = log2(e)·scale·n·(⟨Πq, c⟩ + √(π/2)/d·γ·⟨Sq, s⟩); centroids enter ×64σ.
  const float fk = a.scale * kLog2e / (kCentScale * sigma);
  const float fs = a.scale * kLog2e * 1.2533141373155003f / kD;       // √(π/2)/d
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    qp[j] *= fk;
    qs[j] *= fs;
    m = fmaxf(m, fmaxf(fabsf(qp[j]), fabsf(qs[j])));
  }
  // One power-of-two scale per head for both operands (the split kernel adds
  // the sketch term before scaling back), putting max|·| in [2^9, 2^10).
  m = max4g(m);
  if (g == 0) X.red[1][t][n] = m;
  __syncthreads();
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) m = fmaxf(m, X.red[1][tt][n]);
  int e3 = 0;
  if (m > 0.f) frexpf(m, &e3);
  const float scl = m > 0.f ? ldexpf(1.0f, 10 - e3) : 1.0f;
  // Fragment f (q', K-step f), lane (n, g), slot j holds dim 32g + 8f + j:
  // this wavefront's dims are dwords 2(t%2), 2(t%2) + 1 of fragment t/2.
  uint8_t* blk = a.ws + size_t(unit) * kUnitBytes;
  u32x4* fr = reinterpret_cast<u32x4*>(blk);
  reinterpret_cast<u32x2*>(fr + (t >> 1) * 64 + lane)[t & 1] = hilo_pairs(qp, scl, n < 8);
  if (t == 0 && g == 0 && n < kMaxHeads) reinterpret_cast<float*>(blk + kQFrags * 1024)[n] = live ? 1.0f / scl : 0.f;
  if (prod) {
    // The split kernel's sketch product runs on the scaled fp4 × fp8 matrix
    // cores: its A operand holds -s (fp4 ±1 straight from the sketch bits),
    // so the B operand holds v = -q_S·scl, split into four fp8 parts of four
    // significant bits; part p of (head, 32-coordinate block) is scaled by
    // 2^(S1 - 4p), S1 putting the block's max|v| in [2^7, 2^8). Product 0
    // takes parts 0 (columns 0..7) and 1 (8..15), product 1 parts 2 and 3,
    // so the two products accumulate into columns h and h + 8 like the fp16
    // hi/lo operands. Operand layout (gfx950, 16x16x128): K index k of
    // column c sits in lane c + 16·((k mod 64) / 16), byte (k mod 16) +
    // 16·(k / 64); the E8M0 scale of (column c, block b = k / 32) in lane
    // c + 16b. Coordinate 32g + 4n + m of the sign operand is K index
    // 32g + 8m + n, so this wavefront's coordinate 32g + 4t + j is 32g + 8j + t.
    float v[4], vm = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = -qs[j] * scl;
      vm = fmaxf(vm, fabsf(v[j]));
    }
    X.bmax[t][lane] = vm;
    __syncthreads();
    float M = 0.f;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) M = fmaxf(M, X.bmax[tt][lane]);
    int e = 0;
    if (M > 0.f) frexpf(M, &e);
    const int S1 = M > 0.f ? max(e - 8, -100) : 0;
    uint8_t* sk = blk + kSkOff;
    const int odd = n >= 8 ? 1 : 0;      // this lane's column takes the odd parts
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int S = S1 - 4 * p;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t code = e4m3_rne(ldexpf(v[j], -S));
        v[j] -= ldexpf(e4m3_value(code), S);
        if ((p & 1) == odd) {
          const int k = 32 * g + 8 * j + t;
          const int lb = n + 16 * ((k & 63) >> 4);
          sk[(p >> 1) * 2048 + lb * 32 + (k & 15) + 16 * (k >> 6)] = static_cast<uint8_t>(code);
        }
      }
    }
    if (t == 0) {
      uint32_t* sc = reinterpret_cast<uint32_t*>(blk + kSkScaleOff);
      sc[lane] = static_cast<uint32_t>(127 + S1 - 4 * odd);            // product 0: part odd
      sc[64 + lane] = static_cast<uint32_t>(127 + S1 - 4 * (2 + odd));  // product 1: part 2 + odd
    }
  }
}

__global__ __launch_bounds__(kRowWaves * 64) void query_prep_kernel(PrepArgs a) {
  __shared__ RowXchg X;
  row_prep(a, blockIdx.x, X);
}

// A decode step's small work in one launch: workgroups [0, ktiles) append the
// new keys, the next vtiles the new values (row-tile encoders, one 16-row tile
// each), the last `units` form the query operands.
struct StepArgs {
  PrepArgs prep;
  RowEncArgs kenc, venc;
  int ktiles, vtiles;
};

__global__ __launch_bounds__(kRowWaves * 64) void step_prologue_kernel(StepArgs a) {
  __shared__ RowXchg X;
  const int bid = blockIdx.x;
  if (bid < a.ktiles)
    row_encode(a.kenc, bid, X);
  else if (bid < a.ktiles + a.vtiles)
    row_encode(a.venc, bid - a.ktiles, X);
  else
    row_prep(a.prep, bid - a.ktiles - a.vtiles, X);
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
  const float* kcent_o;   // outlier-channel split: the outlier groups' codebooks
  const float* vcent_o;
};

// W bits at compile-time bit offset OFF of a little-endian word array,
// returned shifted left by SH. The extract is one v_bfe_u32 (an alignbit
// first when the field straddles two words); the shift then folds into the
// address add (v_lshl_add_u32): two operations per table address.
template <int OFF, int W>
__device__ __forceinline__ uint32_t bfe_u32(uint32_t x) {
  return __builtin_amdgcn_ubfe(x, OFF, W);
}

template <int OFF, int W, int SH, int N>
__device__ __forceinline__ uint32_t field_shl(const uint32_t (&w)[N]) {
  constexpr int wi = OFF >> 5, off = OFF & 31;
  if constexpr (off + W <= 32)
    return bfe_u32<off, W>(w[wi]) << SH;
  else
    return bfe_u32<0, W>(__builtin_amdgcn_alignbit(w[wi + 1], w[wi], off)) << SH;
}

// ---- lookup tables in LDS -------------------------------------------------
// Codes index small tables with per-lane addresses. Random lanes hitting one
// LDS bank serialise, so the tables read most often are kept as kCopies
// private copies: copy c = lane % 32 of entry e sits at e·(kCopies·width) +
// c·width, and the 32 lanes of a half-wavefront always read 32 different banks.
constexpr int kCopies = 32;

// The private tables share one 64 KiB region of 256 rows × 256 bytes:
//   value pairs: entry e in row e at byte 4c, c = lane % 32 (the lower half
//     of the row), so that one byte permute forms the address (entry in bits
//     8..15, 4c in bits 0..7);
//   3-bit key pairs: entry e in row e at byte 128 + 4c, c = lane % 32 (the
//     decode kernel replicates them over all 256 rows, row r holding pair
//     r & 63, for byte-permute addresses; the search table has rows 0..63);
//   4-bit key pairs and 2-bit key quads (8-byte entries, indexed by a whole
//     code byte): entry e in row e at byte 128 + 8c', c' = lane % 16 (two
//     lanes of a half-wavefront share a copy), addressed by one byte permute.
// The sketch-nibble table (8 bytes per copy) lives in its own 4 KiB array,
// entry e of copy c at byte 256e + 8c: the upper halves of the rows above
// only reach half of the banks.
constexpr int kTabBytes = 256 * 256;
constexpr uint32_t kTabK = 128;

// Key tables. Each entry covers a group of codes (pairs for 3 and 4 bits,
// quads for 2, octets for 1) and holds their fp16 centroids c·64σ packed in
// pairs; the 4-bit table appends the fp16 remainders (lo parts). The 2-, 3-
// and 4-bit tables are private copies in the shared region; the 1-bit octet
// table is shared by all lanes.
template <int BK> struct KLut {
  static constexpr bool priv = BK >= 2;
  static constexpr bool byte_indexed = BK == 2 || BK == 4;   // 8-byte entries, 16 copies
  static constexpr int per = (BK == 3 || BK == 4) ? 2 : BK == 2 ? 4 : 8;     // codes per entry
  static constexpr int entries = BK == 3 ? 64 : 256;
  static constexpr int dwords = BK == 1 ? 4 : (BK == 2 || BK == 4) ? 2 : 1;  // per entry
  static constexpr int bytes = (BK == 0 || priv) ? 16 : entries * dwords * 4;   // the separate shared table
};

// Byte offset of entry (byte B of w) in a row-per-entry table: the entry in
// bits 8..15, the lane's copy offset (< 256) in bits 0..7; one byte permute.
template <int B>
__device__ __forceinline__ uint32_t row_addr(uint32_t w, uint32_t lane_off) {
  return __builtin_amdgcn_perm(w, lane_off, 0x03020000u | ((4u + B) << 8));
}

// The same for byte B (0..11) of a 96-bit string held in three words.
template <int B>
__device__ __forceinline__ uint32_t byte_addr(const uint32_t (&w)[3], uint32_t lane_off) {
  return row_addr<B & 3>(w[B >> 2], lane_off);
}

// 3-bit keys with the replicated pair table (row r holds pair r & 63, so
// the two bits above a 6-bit field do not matter): pair field f of the lane's
// 96-bit code string starts at bit 6f, i.e. at bit 0, 6, 4 or 2 of a byte for
// f mod 4 = 0, 1, 2, 3. The string shifted right by 6, 4 and 2 bits puts
// every field at the bottom of a byte, and one byte permute per field then
// forms its table address (nine funnel shifts per tile instead of one shift
// per field).
struct KeyShifts {
  uint32_t s6[3], s4[3], s2[3];
};
__device__ __forceinline__ KeyShifts key_shifts(const uint32_t (&w)[3]) {
  KeyShifts k;
  k.s6[0] = __builtin_amdgcn_alignbit(w[1], w[0], 6);
  k.s6[1] = __builtin_amdgcn_alignbit(w[2], w[1], 6);
  k.s6[2] = w[2] >> 6;
  k.s4[0] = __builtin_amdgcn_alignbit(w[1], w[0], 4);
  k.s4[1] = __builtin_amdgcn_alignbit(w[2], w[1], 4);
  k.s4[2] = w[2] >> 4;
  k.s2[0] = __builtin_amdgcn_alignbit(w[1], w[0], 2);
  k.s2[1] = __builtin_amdgcn_alignbit(w[2], w[1], 2);
  k.s2[2] = w[2] >> 2;
  return k;
}

// A operand of K-step S (fields 4S .. 4S + 3, in bytes 3S of the unshifted
// and the 6-shifted string, 3S + 1 of the 4-shifted, 3S + 2 of the
// 2-shifted one) from the replicated 3-bit pair table.
template <int S>
__device__ __forceinline__ u32x4 key_operand3r(const uint32_t (&kw)[3], const KeyShifts& ks, const uint8_t* lut,
                                               uint32_t lane4) {
  u32x4 hi;
  hi[0] = *reinterpret_cast<const uint32_t*>(lut + byte_addr<3 * S>(kw, lane4));
  hi[1] = *reinterpret_cast<const uint32_t*>(lut + byte_addr<3 * S>(ks.s6, lane4));
  hi[2] = *reinterpret_cast<const uint32_t*>(lut + byte_addr<3 * S + 1>(ks.s4, lane4));
  hi[3] = *reinterpret_cast<const uint32_t*>(lut + byte_addr<3 * S + 2>(ks.s2, lane4));
  return hi;
}

// A operands of K-step S from the lane's 32 key codes (hi; lo for 4 bits).
// `lut` is the table; `lane4` the byte offset of the lane's private copy.
template <int BK, int S>
__device__ __forceinline__ void key_operands(const uint32_t (&kw)[BK > 0 ? BK : 1], const uint8_t* lut,
                                             uint32_t lane4, u32x4& hi, u32x4& lo) {
  if constexpr (BK == 4) {
    // entry (pair code byte p of word S) of copy c' at byte 256e + 128 + 8c' (lane4 = 128 + 8c')
    const u32x2 v0 = *reinterpret_cast<const u32x2*>(lut + row_addr<0>(kw[S], lane4));
    const u32x2 v1 = *reinterpret_cast<const u32x2*>(lut + row_addr<1>(kw[S], lane4));
    const u32x2 v2 = *reinterpret_cast<const u32x2*>(lut + row_addr<2>(kw[S], lane4));
    const u32x2 v3 = *reinterpret_cast<const u32x2*>(lut + row_addr<3>(kw[S], lane4));
    hi = u32x4{v0[0], v1[0], v2[0], v3[0]};
    lo = u32x4{v0[1], v1[1], v2[1], v3[1]};
  } else if constexpr (BK == 3) {
    // entry e of copy c at byte 256e + 128 + 4c (lane4 = 128 + 4c)
    hi[0] = *reinterpret_cast<const uint32_t*>(lut + (field_shl<24 * S + 0, 6, 8>(kw) + lane4));
    hi[1] = *reinterpret_cast<const uint32_t*>(lut + (field_shl<24 * S + 6, 6, 8>(kw) + lane4));
    hi[2] = *reinterpret_cast<const uint32_t*>(lut + (field_shl<24 * S + 12, 6, 8>(kw) + lane4));
    hi[3] = *reinterpret_cast<const uint32_t*>(lut + (field_shl<24 * S + 18, 6, 8>(kw) + lane4));
  } else if constexpr (BK == 2) {
    // quads: bytes 2(S%2), 2(S%2) + 1 of word S/2
    const u32x2 q0 = *reinterpret_cast<const u32x2*>(lut + row_addr<2 * (S & 1)>(kw[S >> 1], lane4));
    const u32x2 q1 = *reinterpret_cast<const u32x2*>(lut + row_addr<2 * (S & 1) + 1>(kw[S >> 1], lane4));
    hi = u32x4{q0[0], q0[1], q1[0], q1[1]};
  } else if constexpr (BK == 1) {
    hi = *reinterpret_cast<const u32x4*>(lut + (((kw[0] >> (8 * S)) & 0xffu) << 4));
  }
}

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// (x & m) | o in one v_and_or_b32 (the mask from a scalar register, the
// other constant from a vector register: one scalar operand per instruction).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(o));
  return r;
}

// Sign operand of a sketch word for the scaled fp4 products: nibble m·8 + c
// (dword m, nibble c) holds coordinate 4c + m of the word as fp4 0x2 | bit<<3:
// -1 for a set bit, +1 otherwise, i.e. -s (the query operand holds -q_S).
__device__ __forceinline__ i32x8 sign_operand4(uint32_t w) {
  // ((w << k) & 0x8...8) | 0x2...2: the sign bit moved to bit 3 of each
  // nibble, exponent bits 01 (magnitude 1)
  constexpr uint32_t kSign = 0x88888888u, kOne = 0x22222222u;
  i32x8 v;
  v[0] = static_cast<int32_t>(and_or(w << 3, kSign, kOne));
  v[1] = static_cast<int32_t>(and_or(w << 2, kSign, kOne));
  v[2] = static_cast<int32_t>(and_or(w << 1, kSign, kOne));
  v[3] = static_cast<int32_t>(and_or(w, kSign, kOne));
  v[4] = v[5] = v[6] = v[7] = 0;
  return v;
}

// Value codes of dims 8n..8n+7 → "nibble form": code of dim 8n+r in bits
// [4r, 4r+BV). Spreads 8 fields of BV bits to 4-bit spacing.
template <int BV>
__device__ __forceinline__ uint32_t to_nibbles(uint32_t w) {
  if constexpr (BV == 4) {
    return w;
  } else if constexpr (BV == 3) {
    const uint32_t t = __builtin_amdgcn_ubfe(w, 0, 12) | ((w << 4) & 0x0fff0000u);
    const uint32_t u = (t & 0x003f003fu) | ((t << 2) & 0x3f003f00u);
    return (u & 0x07070707u) | ((u << 1) & 0x70707070u);
  } else if constexpr (BV == 2) {
    const uint32_t t = (w & 0xffu) | ((w << 8) & 0x00ff0000u);
    const uint32_t u = (t & 0x000f000fu) | ((t << 4) & 0x0f000f00u);
    return (u & 0x03030303u) | ((u << 2) & 0x30303030u);
  } else {
    const uint32_t t = (w & 0x0fu) | ((w << 12) & 0x000f0000u);
    const uint32_t u = (t & 0x00030003u) | ((t << 6) & 0x03000300u);
    return (u & 0x01010101u) | ((u << 3) & 0x10101010u);
  }
}

// ---- LDS staging of 32-token blocks ----------------------------------------
// Each wavefront owns a ring of kStages stage buffers. A block's packed data
// is copied HBM → LDS by direct-to-LDS loads (global_load_lds, or the buffer
// form in stage_block_rs: each lane names a source and the wavefront fills
// consecutive LDS, 16 bytes per lane), so the loads for blocks i+1 and i+2
// are in flight while block i is computed, without holding registers. Each
// load instruction reads one array:
// a block's 32 rows of 16·bits bytes take bits/2 wavefront loads plus a
// half-wavefront (32-lane) one when bits is odd. Stage layout (bytes): key
// codes [32][16·BK] | sketch [32][16] | value codes [32][16·BV] (rows
// transposed within each 16-token tile) | key norms [32] | value norms [32] |
// γ [32].
constexpr int kStages = 2;

template <int BITS>
struct RowLoads {
  static constexpr int full = BITS / 2;     // 64-lane loads of 16 bytes per lane
  static constexpr int half = BITS & 1;     // one 32-lane load
};

template <int BK, bool PROD, int BV>
struct Stage {
  static constexpr int kc = 0;
  static constexpr int qj = kc + 512 * BK;
  static constexpr int vc = qj + (PROD ? 512 : 0);
  static constexpr int kn = vc + 512 * BV;
  static constexpr int vn = kn + 128;
  static constexpr int kg = vn + 128;
  static constexpr int bytes = kg + (PROD ? 128 : 0);
  // load instructions per block: codes, sketch (32 lanes), norms and γ (32
  // lanes, 4 bytes each); BV = 0 stages keys only (the value norms' slot stays
  // reserved so that the norm offsets do not move)
  static constexpr int dma = RowLoads<BK>::full + RowLoads<BK>::half + (PROD ? 1 : 0) +
                             RowLoads<BV>::full + RowLoads<BV>::half + 1 + (BV > 0 ? 1 : 0) + (PROD ? 1 : 0);
};

// Row r (0..31) of a staged value block holds token 16(r/16) + 4(r%4) + (r%16)/4,
// so that the four lane groups reading token slots (g, i) hit four bank ranges.
__device__ __forceinline__ uint32_t vrow_token(uint32_t r) {
  const uint32_t sl = r & 15;
  return 16 * (r >> 4) + 4 * (sl & 3) + (sl >> 2);
}

// Per-lane source coordinates of the code loads. Load j of an array covers
// the 16-byte pieces L = 64j + lane of the block: row L / bits, byte 16(L % bits).
struct DmaLane {
  uint32_t ktok[2], kcol[2], koff[2];   // key codes: token, byte in row, byte offset from the block
  uint32_t vtok[2], vcol[2], voff[2];   // value codes (rows transposed within tiles)
  uint32_t ntok;                        // sketch rows, norms and γ: lane % 32
  uint32_t noff, qoff;                  // 4·ntok, 16·ntok
};

template <int BK, int BV>
__device__ __forceinline__ DmaLane dma_lane(int lane) {
  DmaLane d{};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t L = 64 * j + lane;
    if constexpr (BK > 0) {
      d.ktok[j] = L / BK;
      d.kcol[j] = 16 * (L % BK);
      d.koff[j] = 16 * L;
    }
    if constexpr (BV > 0) {
      d.vtok[j] = vrow_token(L / BV);
      d.vcol[j] = 16 * (L % BV);
      d.voff[j] = d.vtok[j] * (16 * BV) + d.vcol[j];
    }
  }
  d.ntok = lane & 31;
  d.noff = 4 * d.ntok;
  d.qoff = 16 * d.ntok;
  return d;
}

// Cache policy of the packed-cache loads: non-temporal. The cache is streamed
// once per launch; kept out of the caches' normal replacement it leaves the
// rotations, the query operands and the partials resident for the small
// kernels around the scan.
constexpr int kStream = 2;

// Issue the direct-to-LDS loads of the block starting at token t0 into `st`
// (a wave-uniform LDS address). Without AL, token indices past `last` are
// clamped to it (those tokens are masked later); with AL every token of the
// block exists.
template <int BK, bool PROD, int BV, bool AL>
__device__ __forceinline__ void stage_block(uint8_t* st, uint32_t t0, uint32_t last, int lane, const DmaLane& d,
                                            const uint8_t* kc, const uint8_t* kq, const uint8_t* vc,
                                            const float* kn, const float* vn, const float* kg) {
  using L = Stage<BK, PROD, BV>;
  using KD = RowLoads<BK>;
  using VD = RowLoads<BV>;
  constexpr int KR = 16 * BK, VR = 16 * BV;
  // Source of a 16-byte piece (token tok, byte col) of an array with rows of
  // RB bytes: with AL the block's first row is a wave-uniform base and the
  // lane part a fixed offset; otherwise the token is clamped to `last`.
  // The lane offsets pass through an empty asm so that the compiler keeps
  // only the 32-bit offsets live across blocks (not one 64-bit pointer per load).
  auto src = [&](const uint8_t* arr, int rb, uint32_t tok, uint32_t col, uint32_t off) -> const uint8_t* {
    if constexpr (AL) {
      asm volatile("" : "+v"(off));
      return arr + size_t(t0) * rb + off;
    } else {
      return arr + size_t(min(t0 + tok, last)) * rb + col;
    }
  };
  auto nsrc = [&](const float* arr) -> const float* {
    if constexpr (AL) {
      uint32_t off = d.ntok;
      asm volatile("" : "+v"(off));
      return arr + t0 + off;
    } else {
      return arr + min(t0 + d.ntok, last);
    }
  };
#pragma unroll
  for (int j = 0; j < KD::full; ++j)
    __builtin_amdgcn_global_load_lds(src(kc, KR, d.ktok[j], d.kcol[j], d.koff[j]), TQ_LDS(st + L::kc + 1024 * j),
                                     16, 0, kStream);
#pragma unroll
  for (int j = 0; j < VD::full; ++j)
    __builtin_amdgcn_global_load_lds(src(vc, VR, d.vtok[j], d.vcol[j], d.voff[j]), TQ_LDS(st + L::vc + 1024 * j),
                                     16, 0, kStream);
  if (lane < 32) {
    constexpr int kj = KD::full, vj = VD::full;
    if constexpr (KD::half)
      __builtin_amdgcn_global_load_lds(src(kc, KR, d.ktok[kj], d.kcol[kj], d.koff[kj]),
                                       TQ_LDS(st + L::kc + 1024 * kj), 16, 0, kStream);
    if constexpr (PROD)
      __builtin_amdgcn_global_load_lds(src(kq, 16, d.ntok, 0, 16 * d.ntok), TQ_LDS(st + L::qj), 16, 0, kStream);
    if constexpr (VD::half)
      __builtin_amdgcn_global_load_lds(src(vc, VR, d.vtok[vj], d.vcol[vj], d.voff[vj]),
                                       TQ_LDS(st + L::vc + 1024 * vj), 16, 0, kStream);
    __builtin_amdgcn_global_load_lds(nsrc(kn), TQ_LDS(st + L::kn), 4, 0, kStream);
    if constexpr (BV > 0) __builtin_amdgcn_global_load_lds(nsrc(vn), TQ_LDS(st + L::vn), 4, 0, kStream);
    if constexpr (PROD) __builtin_amdgcn_global_load_lds(nsrc(kg), TQ_LDS(st + L::kg), 4, 0, kStream);
  }
}

// Buffer resources over one wavefront's token range of each packed array,
// for launches in which every block of the range exists (AL): a block's loads
// then take the lane's 32-bit offset and a scalar offset, with no address
// arithmetic in vector registers. The range is checked by the hardware (an
// access past it would read zeros).
struct StreamRsrc {
  __amdgpu_buffer_rsrc_t kc, kq, vc, kn, vn, kg;
};
constexpr int kRawBufferFlags = 0x00020000;   // 32-bit data format, no swizzle
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), kRawBufferFlags);
}

// stage_block for the AL launches through the buffer resources: `trel` is
// the block's first token relative to the start of the wavefront's range.
template <int BK, bool PROD, int BV>
__device__ __forceinline__ void stage_block_rs(uint8_t* st, uint32_t trel, int lane, const DmaLane& d,
                                               const StreamRsrc& rs) {
  using L = Stage<BK, PROD, BV>;
  using KD = RowLoads<BK>;
  using VD = RowLoads<BV>;
  constexpr uint32_t KR = 16 * BK, VR = 16 * BV;
#pragma unroll
  for (int j = 0; j < KD::full; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.kc, TQ_LDS(st + L::kc + 1024 * j), 16, d.koff[j], trel * KR, 0,
                                             kStream);
#pragma unroll
  for (int j = 0; j < VD::full; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.vc, TQ_LDS(st + L::vc + 1024 * j), 16, d.voff[j], trel * VR, 0,
                                             kStream);
  if (lane < 32) {
    constexpr int kj = KD::full, vj = VD::full;
    if constexpr (KD::half)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.kc, TQ_LDS(st + L::kc + 1024 * kj), 16, d.koff[kj], trel * KR, 0,
                                               kStream);
    if constexpr (PROD)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.kq, TQ_LDS(st + L::qj), 16, d.qoff, trel * 16, 0, kStream);
    if constexpr (VD::half)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.vc, TQ_LDS(st + L::vc + 1024 * vj), 16, d.voff[vj], trel * VR, 0,
                                               kStream);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.kn, TQ_LDS(st + L::kn), 4, d.noff, trel * 4, 0, kStream);
    if constexpr (BV > 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.vn, TQ_LDS(st + L::vn), 4, d.noff, trel * 4, 0, kStream);
    if constexpr (PROD)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.kg, TQ_LDS(st + L::kg), 4, d.noff, trel * 4, 0, kStream);
  }
}

// One lane's registers of a staged block. Score slot j = 4τ + i is token
// 16τ + 4g + i of the block; key tile τ row n is token 16τ + n.
template <int BK, bool PROD, int BV>
struct Block {
  uint32_t kw[2][BK > 0 ? BK : 1];
  uint32_t qw[2];
  float nk[8], gk[8], nv[8];
  uint32_t vw[8];        // value code word holding dims 8n..8n+7 of slot j
  uint32_t vw2[8];       // the following word (3-bit codes that straddle)
};

// Per-lane LDS byte offsets of the staged reads (add the stage base).
struct StageOffsets {
  uint32_t n, k, q, v0, v1;
};

template <int BK, bool PROD, int BV>
__device__ __forceinline__ StageOffsets stage_offsets(int n, int g) {
  using L = Stage<BK, PROD, BV>;
  StageOffsets o;
  o.n = L::kn + 16 * g;
  o.k = L::kc + n * 16 * BK + 4 * BK * g;
  o.q = L::qj + 16 * n + 4 * g;
  const int vword = BV == 4 ? n : BV == 2 ? (n >> 1) : BV == 1 ? (n >> 2) : ((3 * n) >> 2);
  o.v0 = L::vc + g * 16 * BV + 4 * vword;        // slot (g, i) sits in row 4i + g
  o.v1 = o.v0 + 16 * 16 * BV;
  return o;
}

// Read a staged block into registers. The wait for the block's loads (all
// but the newest `pending` loads of this wavefront done) and the wait for the
// LDS reads are inside each asm statement, so no output is used early. The
// reads land asynchronously while later reads of the same statement still use
// their address registers, so every output is early-clobber (never shares a
// register with an input), and no statement has an output that goes unused.
// The statement also reads the LDS word at `ap` into `pw` (the partner
// wavefront's progress; callers without one pass any LDS address).
#define TQ_VMW "s_waitcnt vmcnt(%[pend])\n\tds_read_b32 %[pw], %[ap]\n\t"
#define TQ_NORMS "ds_read_b128 %[n0], %[an]\n\tds_read_b128 %[n1], %[an] offset:64\n\t"
#define TQ_VNORMS "ds_read_b128 %[n2], %[an] offset:128\n\tds_read_b128 %[n3], %[an] offset:192\n\t"
#define TQ_GAMMA "ds_read_b128 %[n4], %[an] offset:256\n\tds_read_b128 %[n5], %[an] offset:320\n\t"
#define TQ_QJ "ds_read2_b32 %[q0], %[aq] offset1:64\n\t"
#define TQ_LGK "s_waitcnt lgkmcnt(0)"

template <int BK, bool PROD, int BV, int PEND>
__device__ __forceinline__ void read_block(Block<BK, PROD, BV>& R, uint32_t sb, const StageOffsets& o, uint32_t ap,
                                           uint32_t& pw) {
  const uint32_t an = sb + o.n, ak = sb + o.k, aq = sb + o.q, av0 = sb + o.v0, av1 = sb + o.v1;
  f32x4 n0, n1, n2, n3, n4, n5;
  u32x2 q0, v0, v1, v2, v3, v4, v5, v6, v7;
  u32x4 ka, kb;         // key words: BK = 4 (two tiles), BK = 2 (both tiles)
  u32x2 k0, k1, k2;     // key words: BK = 3 (word pairs), BK = 1
  // One asm statement per layout: the wait for the block's loads, every read
  // of the stage (norms, γ, sketch, value and key codes), then the wait for
  // the reads, so no output is used early.
#define TQ_VPAIRS(A, B, C)                                                                          \
  "ds_read2_b32 %[v0], %[av0] offset1:" #A "\n\tds_read2_b32 %[v1], %[av0] offset0:" #B " offset1:" #C "\n\t" \
  "ds_read2_b32 %[v2], %[av1] offset1:" #A "\n\tds_read2_b32 %[v3], %[av1] offset0:" #B " offset1:" #C "\n\t"
#define TQ_VPAIRS3                                                                                   \
  "ds_read2_b32 %[v0], %[av0] offset1:1\n\tds_read2_b32 %[v1], %[av0] offset0:48 offset1:49\n\t"     \
  "ds_read2_b32 %[v2], %[av0] offset0:96 offset1:97\n\tds_read2_b32 %[v3], %[av0] offset0:144 offset1:145\n\t" \
  "ds_read2_b32 %[v4], %[av1] offset1:1\n\tds_read2_b32 %[v5], %[av1] offset0:48 offset1:49\n\t"     \
  "ds_read2_b32 %[v6], %[av1] offset0:96 offset1:97\n\tds_read2_b32 %[v7], %[av1] offset0:144 offset1:145\n\t"
#define TQ_KR4 "ds_read_b128 %[ka], %[ak]\n\tds_read_b128 %[kb], %[ak] offset:1024\n\t"
#define TQ_KR3 "ds_read2_b32 %[k0], %[ak] offset1:192\n\tds_read2_b32 %[k1], %[ak] offset0:1 offset1:193\n\t" \
               "ds_read2_b32 %[k2], %[ak] offset0:2 offset1:194\n\t"
#define TQ_KR2 "ds_read2_b64 %[ka], %[ak] offset1:64\n\t"
#define TQ_KR1 "ds_read2_b32 %[k0], %[ak] offset1:64\n\t"
#define TQ_KR0 ""
#define TQ_KO4 , [ka] "=&v"(ka), [kb] "=&v"(kb)
#define TQ_KO3 , [k0] "=&v"(k0), [k1] "=&v"(k1), [k2] "=&v"(k2)
#define TQ_KO2 , [ka] "=&v"(ka)
#define TQ_KO1 , [k0] "=&v"(k0)
#define TQ_KO0
#define TQ_OUT2 [n0] "=&v"(n0), [n1] "=&v"(n1), [pw] "=&v"(pw)
#define TQ_NO3 , [n2] "=&v"(n2), [n3] "=&v"(n3)
#define TQ_NON TQ_NO3
#define TQ_NO0
#define TQ_NR3 TQ_VNORMS
#define TQ_NRN TQ_VNORMS
#define TQ_NR0 ""
#define TQ_VO3 , [v0] "=&v"(v0), [v1] "=&v"(v1), [v2] "=&v"(v2), [v3] "=&v"(v3), \
               [v4] "=&v"(v4), [v5] "=&v"(v5), [v6] "=&v"(v6), [v7] "=&v"(v7)
#define TQ_VON , [v0] "=&v"(v0), [v1] "=&v"(v1), [v2] "=&v"(v2), [v3] "=&v"(v3)
#define TQ_VO0
#define TQ_OUTP , [n4] "=&v"(n4), [n5] "=&v"(n5), [q0] "=&v"(q0)
#define TQ_IN [pend] "n"(PEND), [ap] "v"(ap), [an] "v"(an), [aq] "v"(aq), [av0] "v"(av0), [av1] "v"(av1), [ak] "v"(ak)
#define TQ_K(VP, VS, KB)                                                                           \
  if constexpr (BK == KB) {                                                                        \
    if constexpr (PROD)                                                                            \
      asm volatile(TQ_VMW TQ_NORMS TQ_NR##VS TQ_GAMMA TQ_QJ VP TQ_KR##KB TQ_LGK                    \
                   : TQ_OUT2 TQ_NO##VS TQ_VO##VS TQ_OUTP TQ_KO##KB : TQ_IN : "memory");            \
    else                                                                                           \
      asm volatile(TQ_VMW TQ_NORMS TQ_NR##VS VP TQ_KR##KB TQ_LGK                                   \
                   : TQ_OUT2 TQ_NO##VS TQ_VO##VS TQ_KO##KB : TQ_IN : "memory");                    \
  }
#define TQ_V(VP, VS) TQ_K(VP, VS, 0) TQ_K(VP, VS, 1) TQ_K(VP, VS, 2) TQ_K(VP, VS, 3) TQ_K(VP, VS, 4)
  // slot i is 4 rows (16·BV dwords) after slot i-1; pairs (0, 1) and (2, 3) of each tile
  if constexpr (BV == 3) { TQ_V(TQ_VPAIRS3, 3) }
  if constexpr (BV == 4) { TQ_V(TQ_VPAIRS(64, 128, 192), N) }
  if constexpr (BV == 2) { TQ_V(TQ_VPAIRS(32, 64, 96), N) }
  if constexpr (BV == 1) { TQ_V(TQ_VPAIRS(16, 32, 48), N) }
  if constexpr (BV == 0) { TQ_V("", 0) }
#undef TQ_V
#undef TQ_K
#undef TQ_VPAIRS
#undef TQ_VPAIRS3
#undef TQ_KR4
#undef TQ_KR3
#undef TQ_KR2
#undef TQ_KR1
#undef TQ_KR0
#undef TQ_KO4
#undef TQ_KO3
#undef TQ_KO2
#undef TQ_KO1
#undef TQ_KO0
#undef TQ_OUT2
#undef TQ_NO3
#undef TQ_NON
#undef TQ_NO0
#undef TQ_NR3
#undef TQ_NRN
#undef TQ_NR0
#undef TQ_VO3
#undef TQ_VON
#undef TQ_VO0
#undef TQ_OUTP
#undef TQ_IN
  if constexpr (BK == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) { R.kw[0][k] = ka[k]; R.kw[1][k] = kb[k]; }
  } else if constexpr (BK == 3) {
    R.kw[0][0] = k0[0]; R.kw[1][0] = k0[1];
    R.kw[0][1] = k1[0]; R.kw[1][1] = k1[1];
    R.kw[0][2] = k2[0]; R.kw[1][2] = k2[1];
  } else if constexpr (BK == 2) {
    R.kw[0][0] = ka[0]; R.kw[0][1] = ka[1]; R.kw[1][0] = ka[2]; R.kw[1][1] = ka[3];
  } else if constexpr (BK == 1) {
    R.kw[0][0] = k0[0]; R.kw[1][0] = k0[1];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    R.nk[i] = n0[i]; R.nk[4 + i] = n1[i];
    if constexpr (BV > 0) { R.nv[i] = n2[i]; R.nv[4 + i] = n3[i]; }
    if constexpr (PROD) { R.gk[i] = n4[i]; R.gk[4 + i] = n5[i]; }
  }
  if constexpr (PROD) { R.qw[0] = q0[0]; R.qw[1] = q0[1]; }
  if constexpr (BV == 3) {
    const u32x2 vv[8] = {v0, v1, v2, v3, v4, v5, v6, v7};
#pragma unroll
    for (int j = 0; j < 8; ++j) { R.vw[j] = vv[j][0]; R.vw2[j] = vv[j][1]; }
  } else if constexpr (BV > 0) {
    const u32x2 vv[4] = {v0, v1, v2, v3};
#pragma unroll
    for (int k = 0; k < 4; ++k) { R.vw[2 * k] = vv[k][0]; R.vw[2 * k + 1] = vv[k][1]; }
  }
}
#undef TQ_VMW
#undef TQ_NORMS
#undef TQ_VNORMS
#undef TQ_GAMMA
#undef TQ_QJ
#undef TQ_LGK

// Online softmax state of one lane (its head is column n % 8). The stored
// weights are 2^(s - mk)·n_v with mk = m + log2(nvs): the value-norm scale nvs
// (a power of two, at least twice every value norm seen) keeps them below 2^8
// for fp16, and a partial (mk, l, acc) combines with others through 2^(mk - M)
// alone.
struct SoftmaxState {
  float m;        // reference max of the scores (log2 domain)
  float mk;       // m + knv
  float l;        // Σ 2^(s - mk)·kRoundUp over this lane's tokens (the factor is divided out at the end)
  float nvs;      // value-norm scale 2^knv (wave-uniform); 0 until a nonzero norm is seen
  float knv;
  float nmr;      // log2(kRoundUp) - mk: exponent offset of the rounded weights
};

constexpr float kLazy = 8.0f;   // rescale only when a score exceeds m by more than 2^8

// Add the value of the lane 8 columns over (row rotation by 8 within each
// 16-lane row): column h gets hi + lo of head h.
__device__ __forceinline__ float add_ror8(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
}

// max of 8 values with three v_max3_f32 and one v_max_f32 (no NaN
// canonicalisation: the scores and norms are never signalling NaNs).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max8f(const float (&v)[8]) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(max3f(v[0], v[1], v[2])), "v"(max3f(v[3], v[4], v[5])));
  return max3f(r, v[6], v[7]);
}

struct Luts {
  const uint8_t* k;
  const uint8_t* v;
  uint32_t klane, vlane;   // byte offsets of the lane's private copies
};

// B operand of P·V for dims 8n + r: four dwords, the fp16 pairs of the value
// codes in byte r/2 of X (r even) or Y (r odd), from the private table.
template <int R>
__device__ __forceinline__ u32x4 pv_operand(const uint32_t (&X)[4], const uint32_t (&Y)[4], const Luts& T) {
  // address = (byte R/2 of X or Y) · 256 + 4c: one byte permute; selector
  // bytes: 0 → byte 0 of vlane (4c), 4 + R/2 → that code byte, 2 and 3 →
  // the zero upper bytes of vlane
  constexpr uint32_t sel = 0x03020000u | ((4u + (R >> 1)) << 8);
  u32x4 bv;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t xy = (R & 1) ? Y[k] : X[k];
    bv[k] = *reinterpret_cast<const uint32_t*>(T.v + __builtin_amdgcn_perm(xy, T.vlane, sel));
  }
  return bv;
}

// Scores of a staged block: column n = head n % 8 (hi part for n < 8, lo part
// above); slot j = 4τ + i is token 16τ + 4g + i. The score is sc·iqs.
template <int BK, bool PROD, int BV>
__device__ __forceinline__ void block_scores(const Block<BK, PROD, BV>& R, const Luts& T, const u32x4 (&bq)[4],
                                             const i32x8 (&bs)[2], int ssc0, int ssc1, float (&sc)[8]) {
  // Every table read of both tiles' key operands is issued before the first
  // product, so the block waits for one LDS round trip instead of one per
  // product (the scheduler would otherwise put each read just before its
  // product). The sketch product runs on the scaled fp4 × fp8 matrix cores as
  // in attend_block: A = -s from the sketch word, B = the query's -q_S in
  // four fp8 parts (parts 0/1 into columns 0-15 with scale ssc0, parts 2/3
  // with ssc1), so dq has the hi/lo column halves of the fp16 key product.
  u32x4 kh[2][4], kl[2][4];
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    if constexpr (BK > 0) {
      key_operands<BK, 0>(R.kw[tau], T.k, T.klane, kh[tau][0], kl[tau][0]);
      key_operands<BK, 1>(R.kw[tau], T.k, T.klane, kh[tau][1], kl[tau][1]);
      key_operands<BK, 2>(R.kw[tau], T.k, T.klane, kh[tau][2], kl[tau][2]);
      key_operands<BK, 3>(R.kw[tau], T.k, T.klane, kh[tau][3], kl[tau][3]);
    }
  }
  i32x8 sa[2];
  if constexpr (PROD) {
    sa[0] = sign_operand4(R.qw[0]);
    sa[1] = sign_operand4(R.qw[1]);
  }
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  // u = ⟨q', c⟩ + γ⟨q_S, s⟩ for this lane's part; the row rotation adds the
  // other part, and the key norm and the query scale finish the score.
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    f32x4 dm = f32x4{0.f, 0.f, 0.f, 0.f}, dq = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (BK > 0) {
#pragma unroll
      for (int S = 0; S < 4; ++S) {
        dm = mfma(kh[tau][S], bq[S], dm);
        if constexpr (BK == 4) dm = mfma(kl[tau][S], bq[S], dm);
      }
    }
    if constexpr (PROD) {
      dq = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sa[tau], bs[0], dq, 4, 0, 0, 127, 0, ssc0);
      dq = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sa[tau], bs[1], dq, 4, 0, 0, 127, 0, ssc1);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 4 * tau + i;
      const float u = PROD ? fmaf(R.gk[j], dq[i], dm[i]) : dm[i];
      sc[j] = add_ror8(u) * R.nk[j];       // the score is sc·iqs
    }
  }
}

// LDS stores for the table build, written as asm: the compiler would make a
// plain LDS store wait for every direct-to-LDS load in flight (it cannot tell
// the tables from the stage ring), and the first blocks' loads are issued
// before the build. A build ends with lds_stores_done() before its barrier.
__device__ __forceinline__ void lds_put4(uint32_t addr, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_put1(uint32_t addr, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_stores_done() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// The workgroup barrier after a table build: the build's stores are done
// (lds_stores_done), and no wait for the blocks' loads in flight (a
// __syncthreads would wait for them: they write LDS).
__device__ __forceinline__ void tables_barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// Codebook of up to 16 entries into one VGPR: lane c (c = lane % 16 < K)
// holds entry c.
template <int K>
__device__ __forceinline__ float codebook_lanes(const float* c, int n) {
  float cv[K];
#pragma unroll
  for (int i = 0; i < K; ++i) cv[i] = scalar_load(c + i);
  float v = 0.f;
#pragma unroll
  for (int i = 0; i < K; ++i) v = n == i ? cv[i] : v;
  return v;
}

// a·b rounded to fp32: the opaque copy keeps the product out of a fused
// multiply-add with what follows (the hi/lo split subtracts from it).
__device__ __forceinline__ float mul_rounded(float a, float b) {
  float x = a * b;
  asm("" : "+v"(x));
  return x;
}

// Codebook q of up to 16 entries into lanes 16q .. 16q + K - 1 of v.
template <int K>
__device__ __forceinline__ float codebook_group(const float* c, int q, int lane, float v) {
  float cv[K];
#pragma unroll
  for (int i = 0; i < K; ++i) cv[i] = scalar_load(c + i);
#pragma unroll
  for (int i = 0; i < K; ++i) v = lane == 16 * q + i ? cv[i] : v;
  return v;
}

// v of lane `src` (a lane permute through the LDS crossbar, as asm for the
// same reason as the stores; it waits for its own result). Called with every
// lane active: a permute does not read the registers of inactive lanes.
__device__ __forceinline__ float lane_val(float v, int src) {
  float r;
  asm volatile("ds_bpermute_b32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r) : "v"(src * 4), "v"(v));
  return r;
}

// Fill the lookup tables of a split workgroup (layouts at KLut and kTabBytes)
// from the codebooks scaled by 64σ; every store is 16 bytes (four private
// copies of a 4-byte entry, or two of an 8-byte one). Lane c < 16 of each
// wavefront holds value centroid c in `vcl` and key centroid c in `kcl`, and
// vsig, ksig are the codebook scales σ (all loaded before the first blocks'
// loads: a wait for a load issued after them would also wait for them).
// REP: 3-bit key pairs replicated over all 256 rows (row r holds pair r & 63)
// for the byte-permute addresses of key_operand3r; otherwise rows 0..63.
template <int BK, int BV, bool REP = false>
__device__ __forceinline__ void build_tables(float vcl, float kcl, float vsig, float ksig, uint8_t* tab,
                                             uint8_t* lut_k, int tid, int nthr) {
  using KL = KLut<BK>;
  constexpr int KV = 1 << BV, KK = BK > 0 ? (1 << BK) : 1;
  const uint32_t tb = lds_addr(tab);
  const float vs = kCentScale * vsig;
  auto vcent = [&](int c) { return mul_rounded(lane_val(vcl, c), vs); };
  // value pairs (none for BV = 0, keys only): entry (c0 | c1 << 4) holds the
  // fp16 centroids of codes c0 (low half) and c1, or 0 when a code is out of
  // range
  for (int q = tid; BV > 0 && q < 256 * 8; q += nthr) {
    const int e = q >> 3, c0 = e & 15, c1 = e >> 4;
    const uint32_t p = pack_h2(vcent(c0 & (KV - 1)), vcent(c1 & (KV - 1)));
    const uint32_t w = (c0 < KV && c1 < KV) ? p : 0u;
    lds_put4(tb + 256 * e + 16 * (q & 7), u32x4{w, w, w, w});
  }
  if constexpr (BK > 0) {
    const float ks = kCentScale * ksig;
    auto kcent = [&](int c) { return mul_rounded(lane_val(kcl, c), ks); };
    if constexpr (KL::byte_indexed) {
      // entry e: BK = 4: codes (e & 15, e >> 4), hi pair then lo pair;
      // BK = 2: codes (e >> 2i) & 3, i < 4, as two pairs
      for (int q = tid; q < 256 * 8; q += nthr) {
        const int e = q >> 3;
        uint32_t w0, w1;
        if constexpr (BK == 4) {
          uint16_t h0, l0, h1, l1;
          split_h(kcent(e & 15), h0, l0);
          split_h(kcent(e >> 4), h1, l1);
          w0 = uint32_t(h0) | (uint32_t(h1) << 16);
          w1 = uint32_t(l0) | (uint32_t(l1) << 16);
        } else {
          w0 = pack_h2(kcent(e & 3), kcent((e >> 2) & 3));
          w1 = pack_h2(kcent((e >> 4) & 3), kcent(e >> 6));
        }
        lds_put4(tb + 256 * e + kTabK + 16 * (q & 7), u32x4{w0, w1, w0, w1});
      }
    } else if constexpr (KL::priv) {
      constexpr int rows = (REP && BK == 3) ? 256 : KL::entries;
      for (int q = tid; q < rows * 8; q += nthr) {
        const int r = q >> 3, e = r & (KL::entries - 1);
        const uint32_t w = pack_h2(kcent(e & (KK - 1)), kcent(e >> BK));
        lds_put4(tb + 256 * r + kTabK + 16 * (q & 7), u32x4{w, w, w, w});
      }
    } else {
      // 1 bit: one shared table of octets, entry e = 8 codes (bit i of e)
      const uint32_t w0 = pack_h2(kcent(0), kcent(0)), w1 = pack_h2(kcent(1), kcent(0)),
                     w2 = pack_h2(kcent(0), kcent(1)), w3 = pack_h2(kcent(1), kcent(1));
      for (int e = tid; e < KL::entries; e += nthr) {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pr = (e >> (2 * i)) & 3;
          v[i] = pr == 0 ? w0 : pr == 1 ? w1 : pr == 2 ? w2 : w3;
        }
        lds_put4(lds_addr(lut_k) + 16 * e, v);
      }
    }
  }
}

// read_block for the split-attention kernel: the key and value norms of the
// lane's own tile only (own_off = 0 for tile 0, 64 bytes for tile 1), γ of
// both tiles, and everything else as read_block.
#define TQ_VMW "s_waitcnt vmcnt(%[pend])\n\tds_read_b32 %[pw], %[ap]\n\t"
#define TQ_NORMS "ds_read_b128 %[n0], %[ao]\n\t"
#define TQ_VNORMS "ds_read_b128 %[n2], %[ao] offset:128\n\t"
#define TQ_GAMMA "ds_read_b128 %[n4], %[an] offset:256\n\tds_read_b128 %[n5], %[an] offset:320\n\t"
#define TQ_QJ "ds_read2_b32 %[q0], %[aq] offset1:64\n\t"
#define TQ_LGK "s_waitcnt lgkmcnt(0)"

template <int BK, bool PROD, int BV, int PEND>
__device__ __forceinline__ void read_block_own(Block<BK, PROD, BV>& R, uint32_t sb, const StageOffsets& o, uint32_t own_off,
                                               uint32_t ap, uint32_t& pw) {
  const uint32_t an = sb + o.n, ao = an + own_off, ak = sb + o.k, aq = sb + o.q, av0 = sb + o.v0, av1 = sb + o.v1;
  f32x4 n0, n2, n4, n5;
  u32x2 q0, v0, v1, v2, v3, v4, v5, v6, v7;
  u32x4 ka, kb;         // key words: BK = 4 (two tiles), BK = 2 (both tiles)
  u32x2 k0, k1, k2;     // key words: BK = 3 (word pairs), BK = 1
  // One asm statement per layout: the wait for the block's loads, every read
  // of the stage (norms, γ, sketch, value and key codes), then the wait for
  // the reads, so no output is used early.
#define TQ_VPAIRS(A, B, C)                                                                          \
  "ds_read2_b32 %[v0], %[av0] offset1:" #A "\n\tds_read2_b32 %[v1], %[av0] offset0:" #B " offset1:" #C "\n\t" \
  "ds_read2_b32 %[v2], %[av1] offset1:" #A "\n\tds_read2_b32 %[v3], %[av1] offset0:" #B " offset1:" #C "\n\t"
#define TQ_VPAIRS3                                                                                   \
  "ds_read2_b32 %[v0], %[av0] offset1:1\n\tds_read2_b32 %[v1], %[av0] offset0:48 offset1:49\n\t"     \
  "ds_read2_b32 %[v2], %[av0] offset0:96 offset1:97\n\tds_read2_b32 %[v3], %[av0] offset0:144 offset1:145\n\t" \
  "ds_read2_b32 %[v4], %[av1] offset1:1\n\tds_read2_b32 %[v5], %[av1] offset0:48 offset1:49\n\t"     \
  "ds_read2_b32 %[v6], %[av1] offset0:96 offset1:97\n\tds_read2_b32 %[v7], %[av1] offset0:144 offset1:145\n\t"
#define TQ_KR4 "ds_read_b128 %[ka], %[ak]\n\tds_read_b128 %[kb], %[ak] offset:1024\n\t"
#define TQ_KR3 "ds_read2_b32 %[k0], %[ak] offset1:192\n\tds_read2_b32 %[k1], %[ak] offset0:1 offset1:193\n\t" \
               "ds_read2_b32 %[k2], %[ak] offset0:2 offset1:194\n\t"
#define TQ_KR2 "ds_read2_b64 %[ka], %[ak] offset1:64\n\t"
#define TQ_KR1 "ds_read2_b32 %[k0], %[ak] offset1:64\n\t"
#define TQ_KR0 ""
#define TQ_KO4 , [ka] "=&v"(ka), [kb] "=&v"(kb)
#define TQ_KO3 , [k0] "=&v"(k0), [k1] "=&v"(k1), [k2] "=&v"(k2)
#define TQ_KO2 , [ka] "=&v"(ka)
#define TQ_KO1 , [k0] "=&v"(k0)
#define TQ_KO0
#define TQ_OUT2 [n0] "=&v"(n0), [pw] "=&v"(pw)
#define TQ_NO3 , [n2] "=&v"(n2)
#define TQ_NON TQ_NO3
#define TQ_NO0
#define TQ_NR3 TQ_VNORMS
#define TQ_NRN TQ_VNORMS
#define TQ_NR0 ""
#define TQ_VO3 , [v0] "=&v"(v0), [v1] "=&v"(v1), [v2] "=&v"(v2), [v3] "=&v"(v3), \
               [v4] "=&v"(v4), [v5] "=&v"(v5), [v6] "=&v"(v6), [v7] "=&v"(v7)
#define TQ_VON , [v0] "=&v"(v0), [v1] "=&v"(v1), [v2] "=&v"(v2), [v3] "=&v"(v3)
#define TQ_VO0
#define TQ_OUTP , [n4] "=&v"(n4), [n5] "=&v"(n5), [q0] "=&v"(q0)
#define TQ_IN [pend] "n"(PEND), [ap] "v"(ap), [an] "v"(an), [ao] "v"(ao), [aq] "v"(aq), [av0] "v"(av0), [av1] "v"(av1), [ak] "v"(ak)
#define TQ_K(VP, VS, KB)                                                                           \
  if constexpr (BK == KB) {                                                                        \
    if constexpr (PROD)                                                                            \
      asm volatile(TQ_VMW TQ_NORMS TQ_NR##VS TQ_GAMMA TQ_QJ VP TQ_KR##KB TQ_LGK                    \
                   : TQ_OUT2 TQ_NO##VS TQ_VO##VS TQ_OUTP TQ_KO##KB : TQ_IN : "memory");            \
    else                                                                                           \
      asm volatile(TQ_VMW TQ_NORMS TQ_NR##VS VP TQ_KR##KB TQ_LGK                                   \
                   : TQ_OUT2 TQ_NO##VS TQ_VO##VS TQ_KO##KB : TQ_IN : "memory");                    \
  }
#define TQ_V(VP, VS) TQ_K(VP, VS, 0) TQ_K(VP, VS, 1) TQ_K(VP, VS, 2) TQ_K(VP, VS, 3) TQ_K(VP, VS, 4)
  // slot i is 4 rows (16·BV dwords) after slot i-1; pairs (0, 1) and (2, 3) of each tile
  if constexpr (BV == 3) { TQ_V(TQ_VPAIRS3, 3) }
  if constexpr (BV == 4) { TQ_V(TQ_VPAIRS(64, 128, 192), N) }
  if constexpr (BV == 2) { TQ_V(TQ_VPAIRS(32, 64, 96), N) }
  if constexpr (BV == 1) { TQ_V(TQ_VPAIRS(16, 32, 48), N) }
  if constexpr (BV == 0) { TQ_V("", 0) }
#undef TQ_V
#undef TQ_K
#undef TQ_VPAIRS
#undef TQ_VPAIRS3
#undef TQ_KR4
#undef TQ_KR3
#undef TQ_KR2
#undef TQ_KR1
#undef TQ_KR0
#undef TQ_KO4
#undef TQ_KO3
#undef TQ_KO2
#undef TQ_KO1
#undef TQ_KO0
#undef TQ_OUT2
#undef TQ_NO3
#undef TQ_NON
#undef TQ_NO0
#undef TQ_NR3
#undef TQ_NRN
#undef TQ_NR0
#undef TQ_VO3
#undef TQ_VON
#undef TQ_VO0
#undef TQ_OUTP
#undef TQ_IN
  if constexpr (BK == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) { R.kw[0][k] = ka[k]; R.kw[1][k] = kb[k]; }
  } else if constexpr (BK == 3) {
    R.kw[0][0] = k0[0]; R.kw[1][0] = k0[1];
    R.kw[0][1] = k1[0]; R.kw[1][1] = k1[1];
    R.kw[0][2] = k2[0]; R.kw[1][2] = k2[1];
  } else if constexpr (BK == 2) {
    R.kw[0][0] = ka[0]; R.kw[0][1] = ka[1]; R.kw[1][0] = ka[2]; R.kw[1][1] = ka[3];
  } else if constexpr (BK == 1) {
    R.kw[0][0] = k0[0]; R.kw[1][0] = k0[1];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    R.nk[i] = n0[i];
    if constexpr (BV > 0) R.nv[i] = n2[i];
    if constexpr (PROD) { R.gk[i] = n4[i]; R.gk[4 + i] = n5[i]; }
  }
  if constexpr (PROD) { R.qw[0] = q0[0]; R.qw[1] = q0[1]; }
  if constexpr (BV == 3) {
    const u32x2 vv[8] = {v0, v1, v2, v3, v4, v5, v6, v7};
#pragma unroll
    for (int j = 0; j < 8; ++j) { R.vw[j] = vv[j][0]; R.vw2[j] = vv[j][1]; }
  } else if constexpr (BV > 0) {
    const u32x2 vv[4] = {v0, v1, v2, v3};
#pragma unroll
    for (int k = 0; k < 4; ++k) { R.vw[2 * k] = vv[k][0]; R.vw[2 * k + 1] = vv[k][1]; }
  }
}
#undef TQ_VMW
#undef TQ_NORMS
#undef TQ_VNORMS
#undef TQ_GAMMA
#undef TQ_QJ
#undef TQ_LGK

// The value of lane n ^ 8 (row rotation by 8 within each 16-lane row).
__device__ __forceinline__ float ror8(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
}

// max of 4 values in two instructions (no NaN canonicalisation, as max8f).
__device__ __forceinline__ float max4f(float a, float b, float c, float d) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(max3f(a, b, c)), "v"(d));
  return r;
}

// Full scores of the lane's own tile: lanes n < 8 of each 16-lane row add
// their tile-0 column to that of lane n + 8, lanes n >= 8 their tile-1 column
// to that of lane n - 8 (row rotation by 8; each add writes one half of every
// row through its bank mask). The leading wait covers the DPP read of
// registers just written by vector instructions.
__device__ __forceinline__ void own_tile_sums(const float (&b0)[4], const float (&b1)[4], float (&s)[4]) {
  asm("s_nop 1\n\t"
      "v_add_f32_dpp %0, %4, %4 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %1, %5, %5 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %2, %6, %6 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %3, %7, %7 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %0, %8, %8 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %1, %9, %9 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %2, %10, %10 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %3, %11, %11 row_ror:8 row_mask:0xf bank_mask:0xc"
      : "=&v"(s[0]), "=&v"(s[1]), "=&v"(s[2]), "=&v"(s[3])
      : "v"(b0[0]), "v"(b0[1]), "v"(b0[2]), "v"(b0[3]), "v"(b1[0]), "v"(b1[1]), "v"(b1[2]), "v"(b1[3]));
}

// Weights are formed as 2^(s - mk)·n_v·(1 + 2^-11) and converted to fp16 by
// one round-toward-zero packed conversion: the factor makes the conversion
// round to the nearer of the two neighbours (ties up) instead of toward zero.
constexpr float kRoundUp = 1.0f + 0x1p-11f;
// log2(kRoundUp): the factor is applied as an offset of the exponent, so the
// running sums l carry it too and are divided by kRoundUp at the end.
constexpr float kLog2RoundUp = 7.04269011e-4f;

template <int BK, bool PROD, int BV>
__device__ __forceinline__ void attend_block(const Block<BK, PROD, BV>& R, uint32_t t0, uint32_t t_end, int n, int g,
                                             bool own1, const Luts& T, const u32x4 (&bq)[4], const i32x8 (&bs)[2],
                                             int ssc0, int ssc1, float iqs, SoftmaxState& st, f32x4 (&acc)[8]) {
  // Value codes regrouped for the pair-table addresses: byte q of X holds
  // the codes of slots (2k, 2k+1) for dim 8n + 2q, of Y for dim 8n + 2q + 1.
  uint32_t X[4], Y[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t a0, a1;
    if constexpr (BV == 3) {
      const int off = (24 * n) & 31;
      a0 = to_nibbles<3>(__builtin_amdgcn_alignbit(R.vw2[2 * k], R.vw[2 * k], off));
      a1 = to_nibbles<3>(__builtin_amdgcn_alignbit(R.vw2[2 * k + 1], R.vw[2 * k + 1], off));
    } else if constexpr (BV == 2) {
      a0 = to_nibbles<2>(R.vw[2 * k] >> (16 * (n & 1)));
      a1 = to_nibbles<2>(R.vw[2 * k + 1] >> (16 * (n & 1)));
    } else if constexpr (BV == 1) {
      a0 = to_nibbles<1>(R.vw[2 * k] >> (8 * (n & 3)));
      a1 = to_nibbles<1>(R.vw[2 * k + 1] >> (8 * (n & 3)));
    } else {
      a0 = R.vw[2 * k];
      a1 = R.vw[2 * k + 1];
    }
    X[k] = ((a1 << 4) & 0xf0f0f0f0u) | (a0 & 0x0f0f0f0fu);
    Y[k] = (a1 & 0xf0f0f0f0u) | ((a0 >> 4) & 0x0f0f0f0fu);
  }
  // ---- scores: every key-table read of both tiles goes out before the
  // first product, every product before the first use of a result
  u32x4 kh[2][4], kl[2][4];
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    if constexpr (BK == 3) {
      const KeyShifts ks = key_shifts(R.kw[tau]);
      kh[tau][0] = key_operand3r<0>(R.kw[tau], ks, T.k, T.klane);
      kh[tau][1] = key_operand3r<1>(R.kw[tau], ks, T.k, T.klane);
      kh[tau][2] = key_operand3r<2>(R.kw[tau], ks, T.k, T.klane);
      kh[tau][3] = key_operand3r<3>(R.kw[tau], ks, T.k, T.klane);
    } else if constexpr (BK > 0) {
      key_operands<BK, 0>(R.kw[tau], T.k, T.klane, kh[tau][0], kl[tau][0]);
      key_operands<BK, 1>(R.kw[tau], T.k, T.klane, kh[tau][1], kl[tau][1]);
      key_operands<BK, 2>(R.kw[tau], T.k, T.klane, kh[tau][2], kl[tau][2]);
      key_operands<BK, 3>(R.kw[tau], T.k, T.klane, kh[tau][3], kl[tau][3]);
    }
  }
  i32x8 sa[2];
  if constexpr (PROD) {
    sa[0] = sign_operand4(R.qw[0]);
    sa[1] = sign_operand4(R.qw[1]);
  }
  __builtin_amdgcn_sched_barrier(0);
  f32x4 dm[2], dq[2];
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    dm[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (BK > 0) {
#pragma unroll
      for (int S = 0; S < 4; ++S) {
        dm[tau] = mfma(kh[tau][S], bq[S], dm[tau]);
        if constexpr (BK == 4) dm[tau] = mfma(kl[tau][S], bq[S], dm[tau]);
      }
    }
  }
  if constexpr (PROD) {
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      dq[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
      dq[tau] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sa[tau], bs[0], dq[tau], 4, 0, 0, 127, 0, ssc0);
      dq[tau] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sa[tau], bs[1], dq[tau], 4, 0, 0, 127, 0, ssc1);
    }
  }
  // ---- P·V operands (column n = dim 8n + r, rows = token slots): their
  // table reads run while the products finish
  u32x4 bv[8];
  bv[0] = pv_operand<0>(X, Y, T);
  bv[1] = pv_operand<1>(X, Y, T);
  bv[2] = pv_operand<2>(X, Y, T);
  bv[3] = pv_operand<3>(X, Y, T);
  bv[4] = pv_operand<4>(X, Y, T);
  bv[5] = pv_operand<5>(X, Y, T);
  bv[6] = pv_operand<6>(X, Y, T);
  bv[7] = pv_operand<7>(X, Y, T);
  float br[2][4];
#pragma unroll
  for (int tau = 0; tau < 2; ++tau)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (PROD)
        br[tau][i] = fmaf(R.gk[4 * tau + i], dq[tau][i], dm[tau][i]);
      else
        br[tau][i] = dm[tau][i];
    }
  // Columns h and h + 8 hold the two halves of head h's score (the query's
  // hi and lo parts); lane n takes the full scores of its own tile (tile 0
  // for n < 8, tile 1 for n >= 8) and hands the other tile's half over.
  float sc[4];
  own_tile_sums(br[0], br[1], sc);
#pragma unroll
  for (int i = 0; i < 4; ++i) sc[i] *= R.nk[i];     // the score is sc·iqs
  float nv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) nv[i] = R.nv[i];
  if (__builtin_expect(t0 + kBlockTok > t_end, 0)) {   // last block of the range: mask
    const uint32_t tb = t0 + (own1 ? 16u : 0u) + 4u * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = tb + i < t_end;
      sc[i] = ok ? sc[i] : -INFINITY;
      nv[i] = ok ? nv[i] : 0.f;
    }
  }

  // ---- online softmax (log2 domain), lazily rescaled; lanes n and n ^ 8
  // (the two tiles of head n % 8) share one state ------------------------------
  const float mloc = max4f(sc[0], sc[1], sc[2], sc[3]) * iqs;
  const float nvl = max4f(nv[0], nv[1], nv[2], nv[3]);
  if (__builtin_expect(__any(mloc > st.m + kLazy || nvl > st.nvs), 0)) {
    float mg = max4g(mloc);
    mg = fmaxf(mg, ror8(mg));               // this block's max for the head
    float nvw = max4g(nvl);
    nvw = fmaxf(nvw, ror8(nvw));            // and of the value norms (every lane)
    const float m_new = mg > st.m + kLazy ? mg : st.m;
    float nvs_new = st.nvs, knv_new = st.knv;
    if (nvw > st.nvs) {
      int e;
      frexpf(nvw, &e);                      // nvw < 2^e
      nvs_new = ldexpf(1.0f, e + 1);
      knv_new = static_cast<float>(e + 1);
    }
    const float mk_new = m_new + knv_new;
    const float f = st.mk == -INFINITY ? 0.f : exp2f(st.mk - mk_new);
    st.l *= f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float fi = __shfl(f, (4 * g + i) & 7, 64);   // row 4g+i holds head (4g+i)%8
#pragma unroll
      for (int r = 0; r < 8; ++r) acc[r][i] *= fi;
    }
    st.m = m_new;
    st.mk = mk_new;
    st.nmr = kLog2RoundUp - mk_new;
    st.nvs = nvs_new;
    st.knv = knv_new;
  }
  // A operand of P·V: row n < 8 carries head n's weights of tile 0 (slots
  // 0..3 of each lane group), row n + 8 those of tile 1 (slots 4..7); rows h
  // and h + 8 of the result are summed at the end.
  float w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p = __builtin_amdgcn_exp2f(fmaf(sc[i], iqs, st.nmr));   // 2^(s - mk)·kRoundUp
    st.l += p;
    w[i] = p * nv[i];
  }
  const uint32_t x0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(w[0], w[1]));
  const uint32_t x1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(w[2], w[3]));
  const u32x4 pa = own1 ? u32x4{0u, 0u, x0, x1} : u32x4{x0, x1, 0u, 0u};

  // ---- P·V -------------------------------------------------------------------
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = mfma(pa, bv[r], acc[r]);
}

template <int BK, bool PROD, int BV, bool AL>
__global__ __launch_bounds__(kDecWaves * 64) void attn_split_kernel(AttnArgs a) {
  using SL = Stage<BK, PROD, BV>;
  using KL = KLut<BK>;
  __shared__ __attribute__((aligned(256))) uint8_t tab[kTabBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lut_k[KL::bytes];
  __shared__ float wm[kDecWaves][kMaxHeads], wl[kDecWaves][kMaxHeads];
  __shared__ uint32_t prog[kDecWaves];   // blocks started per wavefront (issue balance)
  // Per wavefront: the stage ring, large enough to hold the 16 x 128 fp32
  // accumulator rows in the epilogue.
  constexpr int kRing = kStages * SL::bytes > 2 * kMaxHeads * kD * 4 ? kStages * SL::bytes : 2 * kMaxHeads * kD * 4;
  __shared__ __attribute__((aligned(16))) uint8_t stage[kDecWaves][kRing];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar token ranges
  const int n = lane & 15, g = lane >> 4;
  const bool own1 = n >= 8;                 // the lane's own tile: tokens 16..31 of each block
  const int split = blockIdx.x, unit = blockIdx.y;
  const int grp = unit % a.ngroups;
  const int kvh = (unit / a.ngroups) % a.Hkv;
  const int b = unit / (a.ngroups * a.Hkv);
  const int gc = min(kMaxHeads, a.G - grp * kMaxHeads);
  constexpr int nthr = kDecWaves * 64;

  // ---- token range of this wavefront; its first two blocks' loads go out
  // before the table build, so their latency hides it ------------------------
  int64_t L = a.max_ctx;
  if (a.ctx_lens) {
    const int64_t l = a.ctx_lens[b];
    L = l < 0 ? 0 : (l > a.max_ctx ? a.max_ctx : l);
  }
  const int64_t per_wave = a.split_len / kDecWaves;
  const int64_t tb = int64_t(split) * a.split_len + wave * per_wave;
  const int64_t te = min(tb + per_wave, L);
  const uint32_t t_begin = static_cast<uint32_t>(tb);
  const uint32_t t_end = te > tb ? static_cast<uint32_t>(te) : t_begin;
  const uint32_t last = L > 0 ? static_cast<uint32_t>(L - 1) : 0u;
  const int64_t base = (int64_t(b) * a.Hkv + kvh) * a.max_ctx;
  const uint8_t* kc = BK > 0 ? a.kc + base * (16 * BK) : a.vc;
  const float* kn = a.kn + base;
  const uint8_t* kq = PROD ? a.kq + base * 16 : a.vc;
  const float* kg = PROD ? a.kg + base : a.kn;
  const uint8_t* vc = a.vc + base * (16 * BV);
  const float* vn = a.vn + base;
  // the codebooks (lane c < 16 holds centroid c) and the query operands
  constexpr int KV = 1 << BV, KK = BK > 0 ? (1 << BK) : 1;
  const float vcl = codebook_lanes<KV>(a.vcent, n);
  const float kcl = BK > 0 ? codebook_lanes<KK>(a.kcent, n) : 0.f;
  const float vsig = scalar_load(&a.vh->sigma), ksig = BK > 0 ? scalar_load(&a.kh->sigma) : 0.f;
  const uint8_t* blk = a.ws + size_t(unit) * kUnitBytes;
  const u32x4* fr = reinterpret_cast<const u32x4*>(blk);
  u32x4 bq[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) bq[s] = fr[s * 64 + lane];
  i32x8 bs[2];
  int ssc0 = 127, ssc1 = 127;
  if constexpr (PROD) {
    const i32x8* sk = reinterpret_cast<const i32x8*>(blk + kSkOff);
    bs[0] = sk[lane];
    bs[1] = sk[64 + lane];
    const int32_t* ss = reinterpret_cast<const int32_t*>(blk + kSkScaleOff);
    ssc0 = ss[lane];
    ssc1 = ss[64 + lane];
  }
  const float iqs = reinterpret_cast<const float*>(blk + kQFrags * 1024)[n & 7];
  asm volatile("" ::: "memory");   // the loads above go out before the blocks' loads
  uint8_t* ring = &stage[wave][0];
  const uint32_t ring_addr = lds_addr(ring);
  const StageOffsets so = stage_offsets<BK, PROD, BV>(n, g);
  const uint32_t own_off = own1 ? 64u : 0u;
  const DmaLane dl = dma_lane<BK, BV>(lane);
  const uint32_t nblk = (t_end - t_begin + kBlockTok - 1) / kBlockTok;
  StreamRsrc rs;
  if constexpr (AL) {
    const uint32_t ntok = nblk * kBlockTok;   // every block of the range exists
    rs.kc = raw_rsrc(kc + size_t(t_begin) * (16 * BK), ntok * (16 * BK));
    rs.kq = raw_rsrc(kq + size_t(t_begin) * 16, PROD ? ntok * 16 : 0u);
    rs.vc = raw_rsrc(vc + size_t(t_begin) * (16 * BV), ntok * (16 * BV));
    rs.kn = raw_rsrc(kn + t_begin, ntok * 4);
    rs.vn = raw_rsrc(vn + t_begin, BV > 0 ? ntok * 4 : 0u);
    rs.kg = raw_rsrc(kg + t_begin, PROD ? ntok * 4 : 0u);
  }
  auto stage_at = [&](uint8_t* st, uint32_t t0) {
    if constexpr (AL)
      stage_block_rs<BK, PROD, BV>(st, t0 - t_begin, lane, dl, rs);
    else
      stage_block<BK, PROD, BV, AL>(st, t0, last, lane, dl, kc, kq, vc, kn, vn, kg);
  };
  if (nblk > 0) stage_at(ring, t_begin);
  if (nblk > 1) stage_at(ring + SL::bytes, t_begin + kBlockTok);

  // ---- lookup tables ---------------------------------------------------------
  build_tables<BK, BV, true>(vcl, kcl, vsig, ksig, tab, lut_k, tid, nthr);
  if (tid < kDecWaves) lds_put1(lds_addr(&prog[tid]), 0u);
  lds_stores_done();
  Luts T;
  const uint32_t cp = lane & 31;            // private copy of this lane
  T.k = KL::priv ? tab : lut_k;
  T.v = tab;
  T.klane = KL::byte_indexed ? kTabK + 8u * (lane & 15) : KL::priv ? kTabK + 4u * cp : 0u;
  T.vlane = 4u * cp;
  tables_barrier();

  SoftmaxState st{-INFINITY, -INFINITY, 0.f, 0.f, 0.f, INFINITY};
  f32x4 acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Block i is read from stage i % kStages; the loads for block i + 2 go
  // into the stage just read.
  // Issue balance: of the two wavefronts on a SIMD (w and w ^ 4), the older
  // one wins issue ties and would finish its share long before the other,
  // leaving its SIMD half idle while the workgroup waits. Each wavefront
  // posts the number of its current block and, when it is ahead of its
  // partner, lowers its priority until the partner catches up.
  const uint32_t prog_own = lds_addr(&prog[wave]), prog_partner = lds_addr(&prog[wave ^ 4]);
  int cur = 0;
  for (uint32_t i = 0; i < nblk; ++i) {
    const uint32_t t0 = t_begin + i * kBlockTok;
    Block<BK, PROD, BV> R;
    const uint32_t sb = ring_addr + cur * SL::bytes;
    lds_put1(prog_own, i);
    uint32_t pw;
    if (i + 1 < nblk)
      read_block_own<BK, PROD, BV, SL::dma>(R, sb, so, own_off, prog_partner, pw);
    else
      read_block_own<BK, PROD, BV, 0>(R, sb, so, own_off, prog_partner, pw);
    if (__builtin_amdgcn_readfirstlane(pw) < i)
      __builtin_amdgcn_s_setprio(0);
    else
      __builtin_amdgcn_s_setprio(1);
    if (i + 2 < nblk) {
      // block i + 2 goes to stage (cur + 2) % kStages: with two stages, the one
      // just read (read_block waited for all of its reads)
      const int nx = (cur + 2) % kStages;
      stage_at(ring + nx * SL::bytes, t0 + 2 * kBlockTok);
    }
    attend_block<BK, PROD, BV>(R, t0, t_end, n, g, own1, T, bq, bs, ssc0, ssc1, iqs, st, acc);
    cur = cur + 1 == kStages ? 0 : cur + 1;
  }
  __builtin_amdgcn_s_setprio(0);
  float l_run = sum4g(st.l);
  l_run += ror8(l_run);                     // both tiles of the head
  l_run *= 1.0f / kRoundUp;

  // ---- merge the workgroup's wavefronts ------------------------------------
  if (g == 0 && n < kMaxHeads) {
    wm[wave][n] = st.mk;
    wl[wave][n] = l_run;
  }
  // The wavefront's stage ring is free now (its last read waited for every
  // load): reuse it for its accumulator (rows 0..7: heads 0..7 over the
  // blocks' tokens 0..15, rows 8..15: over tokens 16..31).
  float* wacc_own = reinterpret_cast<float*>(&stage[wave][0]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * g + i;
#pragma unroll
    for (int r = 0; r < 8; ++r) wacc_own[row * kD + 8 * n + r] = acc[r][i];
  }
  __syncthreads();
  float* part = a.part + ((size_t(unit) * a.nsplit + split) * kMaxHeads) * kPartStride;
  for (int e = tid; e < gc * kD; e += nthr) {
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
        const float* wa = reinterpret_cast<const float*>(&stage[w][0]);
        A = fmaf(fw, wa[head * kD + dim] + wa[(head + 8) * kD + dim], A);
      }
    }
    float* o = part + head * kPartStride;
    o[4 + dim] = A;
    if (dim == 0) {
      o[0] = M;
      o[1] = Ls;
    }
  }
}

// ---------------------------------------------------------------------------
// 2b. Decode attention over outlier-channel split caches
// ---------------------------------------------------------------------------
// Keys and values quantized with the outlier-channel split ("TurboQuant của
// Google…" (omelet.tech), section "Thực nghiệm: 3.5 bit…"): code-string
// position p holds an outlier coordinate (BK + 1 or BV + 1 bits) when
// p mod 8 < 2 and a regular one (BK or BV bits) otherwise, and each vector
// has a norm per group. The block-structured rotations keep the query prep and
// the merge unchanged; here the positions line up with the matrix-core
// operands:
//   * a key tile's K-step S covers positions 32g + 8S + j of lane group g:
//     elements j = 0, 1 (the first dword of the A operand) are outliers, so
//     the scores take two products per K-step, one with only the outlier
//     dword and one with the three regular dwords, weighted by the token's
//     outlier and regular key norms;
//   * the P·V product r covers positions 8n + r of column n: r = 0, 1 are
//     outliers, so products 0 and 1 take the weights p·n_o and the others
//     p·n_r, with no extra product.
// The staged block is the 32 tokens' code strings as they lie in memory
// (rows of 16·b + 4 bytes, copied as dwords), followed by the norm pairs.
// Prod keys (PROD) add the 32 tokens' sketch words (16 bytes each) and their
// (γ_o, γ_r) pairs.
template <int BK, int BV, bool PROD = false>
struct OStage {
  static constexpr int KR = 16 * BK + 4, VR = 16 * BV + 4;   // code bytes per token
  static constexpr int kc = 0;
  static constexpr int vc = 32 * KR;
  static constexpr int kn = vc + 32 * VR;                     // 32 × (n_o, n_r)
  static constexpr int vn = kn + 256;
  static constexpr int qs = vn + 256;                         // PROD: 32 × 16 sketch bytes
  static constexpr int kg = qs + 512;                         // PROD: 32 × (γ_o, γ_r)
  static constexpr int bytes = PROD ? kg + 256 : vn + 256;
  static constexpr int kdw = 8 * KR, vdw = 8 * VR;            // dwords of the block's codes
  static constexpr int kld = (kdw + 63) / 64, vld = (vdw + 63) / 64;
  static constexpr int dma = kld + vld + 2 + (PROD ? 3 : 0);  // load instructions per block
  static_assert(kn % 16 == 0, "norm pairs are read as 16-byte vectors");
};

// Issue the block's direct-to-LDS dword loads. Without AL, dwords past the
// last token's row (or norm pair) are clamped to the last one of it.
template <int BK, int BV, bool AL, bool PROD = false>
__device__ __forceinline__ void ostage_block(uint8_t* st, uint32_t t0, uint32_t last, int lane, const uint8_t* kc,
                                             const uint8_t* vc, const float* kn, const float* vn,
                                             const uint8_t* kq = nullptr, const float* kg = nullptr) {
  using L = OStage<BK, BV, PROD>;
  const uint32_t ntok = last + 1 - t0;   // tokens of the block that exist (AL: at least 32)
  const uint32_t* ks = reinterpret_cast<const uint32_t*>(kc + size_t(t0) * L::KR);
  const uint32_t* vs = reinterpret_cast<const uint32_t*>(vc + size_t(t0) * L::VR);
  const uint32_t klim = AL ? 0u : ntok * (L::KR / 4) - 1u, vlim = AL ? 0u : ntok * (L::VR / 4) - 1u;
#pragma unroll
  for (int j = 0; j < L::kld; ++j) {
    const uint32_t i = 64u * j + lane;
    if (j + 1 < L::kld || (L::kdw % 64) == 0 || i < uint32_t(L::kdw))
      __builtin_amdgcn_global_load_lds(ks + (AL ? i : min(i, klim)), TQ_LDS(st + L::kc + 256 * j), 4, 0, kStream);
  }
#pragma unroll
  for (int j = 0; j < L::vld; ++j) {
    const uint32_t i = 64u * j + lane;
    if (j + 1 < L::vld || (L::vdw % 64) == 0 || i < uint32_t(L::vdw))
      __builtin_amdgcn_global_load_lds(vs + (AL ? i : min(i, vlim)), TQ_LDS(st + L::vc + 256 * j), 4, 0, kStream);
  }
  const uint32_t nl = AL ? uint32_t(lane) : min(uint32_t(lane), 2u * ntok - 1u);
  __builtin_amdgcn_global_load_lds(kn + 2 * size_t(t0) + nl, TQ_LDS(st + L::kn), 4, 0, kStream);
  __builtin_amdgcn_global_load_lds(vn + 2 * size_t(t0) + nl, TQ_LDS(st + L::vn), 4, 0, kStream);
  if constexpr (PROD) {
    // sketch words (4 per token) and γ pairs, clamped like the rest
    const uint32_t* qsrc = reinterpret_cast<const uint32_t*>(kq + size_t(t0) * 16);
    const uint32_t qlim = AL ? 0u : ntok * 4u - 1u;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t i = 64u * j + lane;
      __builtin_amdgcn_global_load_lds(qsrc + (AL ? i : min(i, qlim)), TQ_LDS(st + L::qs + 256 * j), 4, 0, kStream);
    }
    __builtin_amdgcn_global_load_lds(kg + 2 * size_t(t0) + nl, TQ_LDS(st + L::kg), 4, 0, kStream);
  }
}

// One lane's registers of a staged split block: its key words of both tiles
// (lane group g's 32 positions, aligned to bit 0), the 8 slots' norm pairs and
// value words (column n's 8 positions, aligned to bit 0).
struct OBlock {
  uint32_t kw[2][4];
  float nko[8], nkr[8];    // key norm pairs of the 8 slots (both tiles)
  float nvo[4], nvr[4];    // value norm pairs of the lane's own tile's 4 slots
  uint32_t vw[8];
  uint32_t qw[2];          // prod keys: sketch word g of tokens n and 16 + n
  float gko[8], gkr[8];    // prod keys: the slots' scaled γ_o and γ_r, see oread_prod
};

struct OOffsets {
  uint32_t k, n, v;          // byte offsets in the stage
  uint32_t kshift, vshift;   // bit offsets of the lane's key / value bits in their first dword
};

template <int BK, int BV>
__device__ __forceinline__ OOffsets ostage_offsets(int n, int g) {
  using L = OStage<BK, BV>;
  constexpr int KSB = 4 * BK + 1;          // bytes of a lane group's 32 key positions
  constexpr int VCH = 8 * BV + 2;          // bits of a column's 8 value positions
  OOffsets o;
  o.k = L::kc + n * L::KR + 4 * ((g * KSB) >> 2);
  o.kshift = 8 * ((g * KSB) & 3);
  o.n = L::kn + 32 * g;
  o.v = L::vc + 4 * g * L::VR + 4 * ((n * VCH) >> 5);
  o.vshift = (n * VCH) & 31;
  return o;
}

// Read a staged split block into registers: wait for its loads (all but the
// newest PEND of this wavefront), every read of the stage, then the wait for
// the reads, in one statement with early-clobber outputs. The value norms
// are read for the lane's own tile only (own_off: 0 for tile 0, 128 bytes
// for tile 1); the key norms for both, since each lane forms column parts of
// both tiles' scores.
template <int BK, int BV, int PEND>
__device__ __forceinline__ void oread_block(OBlock& R, uint32_t sb, const OOffsets& o, uint32_t own_off, uint32_t ap,
                                            uint32_t& pw) {
  using L = OStage<BK, BV>;
  constexpr int KT = 4 * L::KR;            // dwords between the two key tiles (16 rows)
  constexpr int VT = L::VR / 4;            // dwords between consecutive tokens
  static_assert(KT + 3 <= 255 && 19 * VT + 1 <= 255, "read2 offsets");
  const uint32_t ak = sb + o.k, an = sb + o.n, av = sb + o.v, ao = an + own_off;
  u32x2 k0, k1, k2, k3;
  f32x4 n0, n1, n2, n3, m0, m1;
  u32x2 v0, v1, v2, v3, v4, v5, v6, v7;
  // slot (τ, i) is token 16τ + 4g + i: dword offset (16τ + i)·VT
  asm volatile(
      "s_waitcnt vmcnt(%[pend])\n\t"
      "ds_read_b32 %[pw], %[ap]\n\t"
      "ds_read2_b32 %[k0], %[ak] offset1:1\n\t"
      "ds_read2_b32 %[k1], %[ak] offset0:2 offset1:3\n\t"
      "ds_read2_b32 %[k2], %[ak] offset0:%[kt0] offset1:%[kt1]\n\t"
      "ds_read2_b32 %[k3], %[ak] offset0:%[kt2] offset1:%[kt3]\n\t"
      "ds_read_b128 %[n0], %[an]\n\t"
      "ds_read_b128 %[n1], %[an] offset:16\n\t"
      "ds_read_b128 %[n2], %[an] offset:128\n\t"
      "ds_read_b128 %[n3], %[an] offset:144\n\t"
      "ds_read_b128 %[m0], %[ao] offset:256\n\t"
      "ds_read_b128 %[m1], %[ao] offset:272\n\t"
      "ds_read2_b32 %[v0], %[av] offset0:%[s0] offset1:%[s0b]\n\t"
      "ds_read2_b32 %[v1], %[av] offset0:%[s1] offset1:%[s1b]\n\t"
      "ds_read2_b32 %[v2], %[av] offset0:%[s2] offset1:%[s2b]\n\t"
      "ds_read2_b32 %[v3], %[av] offset0:%[s3] offset1:%[s3b]\n\t"
      "ds_read2_b32 %[v4], %[av] offset0:%[s4] offset1:%[s4b]\n\t"
      "ds_read2_b32 %[v5], %[av] offset0:%[s5] offset1:%[s5b]\n\t"
      "ds_read2_b32 %[v6], %[av] offset0:%[s6] offset1:%[s6b]\n\t"
      "ds_read2_b32 %[v7], %[av] offset0:%[s7] offset1:%[s7b]\n\t"
      "s_waitcnt lgkmcnt(0)"
      : [k0] "=&v"(k0), [k1] "=&v"(k1), [k2] "=&v"(k2), [k3] "=&v"(k3), [n0] "=&v"(n0), [n1] "=&v"(n1),
        [n2] "=&v"(n2), [n3] "=&v"(n3), [m0] "=&v"(m0), [m1] "=&v"(m1),
        [v0] "=&v"(v0), [v1] "=&v"(v1), [v2] "=&v"(v2), [v3] "=&v"(v3), [v4] "=&v"(v4), [v5] "=&v"(v5),
        [v6] "=&v"(v6), [v7] "=&v"(v7), [pw] "=&v"(pw)
      : [pend] "n"(PEND), [ap] "v"(ap), [ak] "v"(ak), [an] "v"(an), [ao] "v"(ao), [av] "v"(av), [kt0] "n"(KT),
        [kt1] "n"(KT + 1),
        [kt2] "n"(KT + 2), [kt3] "n"(KT + 3), [s0] "n"(0), [s0b] "n"(1), [s1] "n"(VT), [s1b] "n"(VT + 1),
        [s2] "n"(2 * VT), [s2b] "n"(2 * VT + 1), [s3] "n"(3 * VT), [s3b] "n"(3 * VT + 1), [s4] "n"(16 * VT),
        [s4b] "n"(16 * VT + 1), [s5] "n"(17 * VT), [s5b] "n"(17 * VT + 1), [s6] "n"(18 * VT),
        [s6b] "n"(18 * VT + 1), [s7] "n"(19 * VT), [s7b] "n"(19 * VT + 1)
      : "memory");
  const uint32_t ks = o.kshift, vs = o.vshift;
  const u32x2 kk[2][2] = {{k0, k1}, {k2, k3}};
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint32_t d0 = kk[t][0][0], d1 = kk[t][0][1], d2 = kk[t][1][0], d3 = kk[t][1][1];
    R.kw[t][0] = __builtin_amdgcn_alignbit(d1, d0, ks);
    R.kw[t][1] = __builtin_amdgcn_alignbit(d2, d1, ks);
    R.kw[t][2] = __builtin_amdgcn_alignbit(d3, d2, ks);
    R.kw[t][3] = d3 >> ks;
  }
  const f32x4 nn[4] = {n0, n1, n2, n3}, mm[2] = {m0, m1};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    R.nko[j] = nn[j >> 1][2 * (j & 1)];
    R.nkr[j] = nn[j >> 1][2 * (j & 1) + 1];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    R.nvo[i] = mm[i >> 1][2 * (i & 1)];
    R.nvr[i] = mm[i >> 1][2 * (i & 1) + 1];
  }
  const u32x2 vv[8] = {v0, v1, v2, v3, v4, v5, v6, v7};
#pragma unroll
  for (int j = 0; j < 8; ++j) R.vw[j] = __builtin_amdgcn_alignbit(vv[j][1], vv[j][0], vs);
}

// Prod keys: the lane's sketch words of both tiles (word g of tokens n and
// 16 + n) and the 8 slots' γ pairs. The query's sketch operand carries the
// correction scale √(π/2)/128 of a whole vector; a group's estimate takes
// √(π/2)/d_g, i.e. γ_o·128/32 and γ_r·128/96: the factor 4 is applied as
// +2 in the sketch products' E8M0 scales, the remaining 1/3 here.
template <int BK, int BV>
__device__ __forceinline__ void oread_prod(OBlock& R, uint32_t sb, int n, int g) {
  using L = OStage<BK, BV, true>;
  const uint32_t aq = sb + L::qs + 16 * n + 4 * g, ag = sb + L::kg + 32 * g;
  uint32_t q0, q1;
  f32x4 g0, g1, g2, g3;
  asm volatile(
      "ds_read_b32 %[q0], %[aq]\n\t"
      "ds_read_b32 %[q1], %[aq] offset:256\n\t"
      "ds_read_b128 %[g0], %[ag]\n\t"
      "ds_read_b128 %[g1], %[ag] offset:16\n\t"
      "ds_read_b128 %[g2], %[ag] offset:128\n\t"
      "ds_read_b128 %[g3], %[ag] offset:144\n\t"
      "s_waitcnt lgkmcnt(0)"
      : [q0] "=&v"(q0), [q1] "=&v"(q1), [g0] "=&v"(g0), [g1] "=&v"(g1), [g2] "=&v"(g2), [g3] "=&v"(g3)
      : [aq] "v"(aq), [ag] "v"(ag)
      : "memory");
  R.qw[0] = q0;
  R.qw[1] = q1;
  const f32x4 gg[4] = {g0, g1, g2, g3};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    R.gko[j] = gg[j >> 1][2 * (j & 1)];
    R.gkr[j] = gg[j >> 1][2 * (j & 1) + 1] * (1.0f / 3.0f);
  }
}

// Table rows of the split decode (the value pair tables fill the lower and the
// upper half of rows 0..127; rows 128.. of the upper half hold key pairs):
//   outlier value pairs  row e, byte 4c              (e = code0 | code1 << 4)
//   regular value pairs  row e, byte 128 + 4c        (e <= 0x77)
//   regular key pairs    row 128 + e, byte 128 + 4c  (e = 2·BK bits)
//   3-bit outlier key pairs  row 192 + e, byte 128 + 4c
// 4-bit outlier key pairs (hi and lo pairs, 8 bytes) have rows of their own
// (128 bytes, 16 copies: row e, byte 8c').
constexpr int kKeyRegRow = 128, kKeyOutRow = 192;

template <int BK, int S>
// A operand of K-step S: the outlier pair (hi part) in dword 0 and the three
// regular pairs in dwords 1..3; for 4-bit outlier codes `aol` holds the lo
// part of the outlier pair in dword 0 (zeros elsewhere).
__device__ __forceinline__ void okey_operands(const uint32_t (&kw)[4], const uint8_t* tab, const uint8_t* tab2,
                                              uint32_t lane_hi, uint32_t lane8, u32x4& af, u32x4& aol) {
  constexpr int BKO = BK + 1, CH = 8 * BK + 2, base = S * CH;
  if constexpr (BKO == 4) {
    const u32x2 e = *reinterpret_cast<const u32x2*>(tab2 + (field_shl<base, 8, 7>(kw) + lane8));
    af[0] = e[0];
    aol = u32x4{e[1], 0u, 0u, 0u};
  } else {
    af[0] = *reinterpret_cast<const uint32_t*>(tab + kKeyOutRow * 256 + (field_shl<base, 2 * BKO, 8>(kw) + lane_hi));
  }
  const uint8_t* kb = tab + kKeyRegRow * 256;
  af[1] = *reinterpret_cast<const uint32_t*>(kb + (field_shl<base + 2 * BKO, 2 * BK, 8>(kw) + lane_hi));
  af[2] = *reinterpret_cast<const uint32_t*>(kb + (field_shl<base + 2 * BKO + 2 * BK, 2 * BK, 8>(kw) + lane_hi));
  af[3] = *reinterpret_cast<const uint32_t*>(kb + (field_shl<base + 2 * BKO + 4 * BK, 2 * BK, 8>(kw) + lane_hi));
}

// Column n's parts of a split block's scores (head n % 8; columns h and
// h + 8 hold the query's hi and lo parts, and their sum times iqs is the
// score). The two products per K-step
// take the whole A operand against the query split by position: `bqo` keeps
// the outlier slots (dword 0 of each fragment) and `bqr` the regular ones,
// so no A operand needs masking (zero slots contribute exact zeros).
//
// Prod keys add each group's sketch product on the scaled fp4 × fp8 matrix
// cores (as attn_split_kernel's): `bso` holds the query's sketch operand with
// only the outlier positions kept, `bsr` with only the regular ones.
template <int BK, bool PROD>
__device__ __forceinline__ void oblock_scores(const OBlock& R, const uint8_t* tab, const uint8_t* tab2,
                                              uint32_t lane_hi, uint32_t lane8, const u32x4 (&bqo)[4],
                                              const u32x4 (&bqr)[4], const i32x8 (&bso)[2], const i32x8 (&bsr)[2],
                                              int ssc0, int ssc1, float (&sc)[8]) {
  u32x4 af[2][4], aol[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    okey_operands<BK, 0>(R.kw[t], tab, tab2, lane_hi, lane8, af[t][0], aol[t][0]);
    okey_operands<BK, 1>(R.kw[t], tab, tab2, lane_hi, lane8, af[t][1], aol[t][1]);
    okey_operands<BK, 2>(R.kw[t], tab, tab2, lane_hi, lane8, af[t][2], aol[t][2]);
    okey_operands<BK, 3>(R.kw[t], tab, tab2, lane_hi, lane8, af[t][3], aol[t][3]);
  }
  i32x8 sa[2];
  if constexpr (PROD) {
    sa[0] = sign_operand4(R.qw[0]);
    sa[1] = sign_operand4(R.qw[1]);
  }
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f32x4 dmo = f32x4{0.f, 0.f, 0.f, 0.f}, dmr = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int S = 0; S < 4; ++S) {
      dmo = mfma(af[t][S], bqo[S], dmo);
      if constexpr (BK + 1 == 4) dmo = mfma(aol[t][S], bqo[S], dmo);
      dmr = mfma(af[t][S], bqr[S], dmr);
    }
    if constexpr (PROD) {
      f32x4 dqo = f32x4{0.f, 0.f, 0.f, 0.f}, dqr = f32x4{0.f, 0.f, 0.f, 0.f};
      dqo = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sa[t], bso[0], dqo, 4, 0, 0, 127, 0, ssc0);
      dqo = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sa[t], bso[1], dqo, 4, 0, 0, 127, 0, ssc1);
      dqr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sa[t], bsr[0], dqr, 4, 0, 0, 127, 0, ssc0);
      dqr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sa[t], bsr[1], dqr, 4, 0, 0, 127, 0, ssc1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dmo[i] = fmaf(R.gko[4 * t + i], dqo[i], dmo[i]);
        dmr[i] = fmaf(R.gkr[4 * t + i], dqr[i], dmr[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 4 * t + i;
      sc[j] = fmaf(R.nko[j], dmo[i], R.nkr[j] * dmr[i]);   // column n's part of slot j's score
    }
  }
}

// Value positions 8n..8n+7 of a slot in nibble form (code of position 8n + r
// in bits 4r..4r+3): the two outlier codes (BV + 1 bits) then six regular ones.
template <int BV>
__device__ __forceinline__ uint32_t onibbles(uint32_t w) {
  constexpr int BVO = BV + 1;
  const uint32_t o = bfe_u32<0, BVO>(w) | (bfe_u32<BVO, BVO>(w) << 4);
  return o | (to_nibbles<BV>(w >> (2 * BVO)) << 8);
}

template <int BK, int BV, bool PROD>
__device__ __forceinline__ void oattend_block(const OBlock& R, uint32_t t0, uint32_t t_end, int n, int g,
                                              const uint8_t* tab, const uint8_t* tab2, uint32_t lane_lo,
                                              uint32_t lane_hi, uint32_t lane8, const u32x4 (&bqo)[4],
                                              const u32x4 (&bqr)[4], const i32x8 (&bso)[2],
                                              const i32x8 (&bsr)[2], int ssc0, int ssc1, float iqs,
                                              bool own1, SoftmaxState& st, f32x4 (&acc)[8]) {
  uint32_t X[4], Y[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t a0 = onibbles<BV>(R.vw[2 * k]), a1 = onibbles<BV>(R.vw[2 * k + 1]);
    X[k] = (a0 & 0x0f0f0f0fu) | ((a1 << 4) & 0xf0f0f0f0u);
    Y[k] = ((a0 >> 4) & 0x0f0f0f0fu) | (a1 & 0xf0f0f0f0u);
  }
  float part[8];
  oblock_scores<BK, PROD>(R, tab, tab2, lane_hi, lane8, bqo, bqr, bso, bsr, ssc0, ssc1, part);
  Luts Tv;
  Tv.v = tab;
  Tv.vlane = lane_lo;
  u32x4 bv[8];
  bv[0] = pv_operand<0>(X, Y, Tv);
  bv[1] = pv_operand<1>(X, Y, Tv);
  Tv.vlane = lane_hi;
  bv[2] = pv_operand<2>(X, Y, Tv);
  bv[3] = pv_operand<3>(X, Y, Tv);
  bv[4] = pv_operand<4>(X, Y, Tv);
  bv[5] = pv_operand<5>(X, Y, Tv);
  bv[6] = pv_operand<6>(X, Y, Tv);
  bv[7] = pv_operand<7>(X, Y, Tv);
  // Each lane finishes the scores of its own 16-token tile (tile 0 for
  // n < 8, tile 1 for n >= 8), taking the other column half of them from
  // lane n ^ 8, as in attn_split_kernel.
  float sc[4], nvo[4], nvr[4];
  const float pt0[4] = {part[0], part[1], part[2], part[3]}, pt1[4] = {part[4], part[5], part[6], part[7]};
  own_tile_sums(pt0, pt1, sc);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    nvo[i] = R.nvo[i];
    nvr[i] = R.nvr[i];
  }
  if (__builtin_expect(t0 + kBlockTok > t_end, 0)) {
    const uint32_t tb = t0 + (own1 ? 16u : 0u) + 4u * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = tb + i < t_end;
      sc[i] = ok ? sc[i] : -INFINITY;
      nvo[i] = ok ? nvo[i] : 0.f;
      nvr[i] = ok ? nvr[i] : 0.f;
    }
  }
  const float mloc = max4f(sc[0], sc[1], sc[2], sc[3]) * iqs;
  const float nvl = fmaxf(max4f(nvo[0], nvo[1], nvo[2], nvo[3]), max4f(nvr[0], nvr[1], nvr[2], nvr[3]));
  if (__builtin_expect(__any(mloc > st.m + kLazy || nvl > st.nvs), 0)) {
    float mg = max4g(mloc);
    mg = fmaxf(mg, ror8(mg));               // this block's max for the head
    float nvw = max4g(nvl);
    nvw = fmaxf(nvw, ror8(nvw));            // and of the value norms (every lane)
    const float m_new = mg > st.m + kLazy ? mg : st.m;
    float nvs_new = st.nvs, knv_new = st.knv;
    if (nvw > st.nvs) {
      int e;
      frexpf(nvw, &e);
      nvs_new = ldexpf(1.0f, e + 1);
      knv_new = static_cast<float>(e + 1);
    }
    const float mk_new = m_new + knv_new;
    const float f = st.mk == -INFINITY ? 0.f : exp2f(st.mk - mk_new);
    st.l *= f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float fi = __shfl(f, (4 * g + i) & 7, 64);   // row 4g+i holds head (4g+i)%8
#pragma unroll
      for (int r = 0; r < 8; ++r) acc[r][i] *= fi;
    }
    st.m = m_new;
    st.mk = mk_new;
    st.nmr = kLog2RoundUp - mk_new;
    st.nvs = nvs_new;
    st.knv = knv_new;
  }
  // A operands of P·V: weights p·n_o for the outlier products (r = 0, 1),
  // p·n_r for the others, as fp16 rounded to nearest (kRoundUp); row n < 8
  // carries head n's weights of tile 0, row n + 8 those of tile 1, and rows h
  // and h + 8 of the result are summed at the end.
  float wo[4], wr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p = __builtin_amdgcn_exp2f(fmaf(sc[i], iqs, st.nmr));   // 2^(s - mk)·kRoundUp
    st.l += p;
    wo[i] = p * nvo[i];
    wr[i] = p * nvr[i];
  }
  const uint32_t xo0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(wo[0], wo[1]));
  const uint32_t xo1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(wo[2], wo[3]));
  const uint32_t xr0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(wr[0], wr[1]));
  const uint32_t xr1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(wr[2], wr[3]));
  const u32x4 pao = own1 ? u32x4{0u, 0u, xo0, xo1} : u32x4{xo0, xo1, 0u, 0u};
  const u32x4 par = own1 ? u32x4{0u, 0u, xr0, xr1} : u32x4{xr0, xr1, 0u, 0u};
  acc[0] = mfma(pao, bv[0], acc[0]);
  acc[1] = mfma(pao, bv[1], acc[1]);
#pragma unroll
  for (int r = 2; r < 8; ++r) acc[r] = mfma(par, bv[r], acc[r]);
}

// The workgroup's partials of a split (as in attn_split_kernel), with each
// head's rows of tile-0 and tile-1 weights (lane groups g and g + 2) added
// before they are staged, so a wavefront stages 8 rows of 128 floats (4 KiB).
// Lanes n and n ^ 8 hold the running sums of the two tiles of head n % 8.
template <int RING>
__device__ __forceinline__ void write_partials_o(const AttnArgs& a, const SoftmaxState& st, const f32x4 (&acc)[8],
                                                 float (&wm)[kDecWaves][kMaxHeads], float (&wl)[kDecWaves][kMaxHeads],
                                                 uint8_t (&stage)[kDecWaves][RING], int unit, int split, int gc,
                                                 int n, int g, int wave, int tid) {
  static_assert(RING >= kMaxHeads * kD * 4, "accumulator rows");
  float l_run = sum4g(st.l);
  l_run += ror8(l_run);
  l_run *= 1.0f / kRoundUp;
  if (g == 0 && n < kMaxHeads) {
    wm[wave][n] = st.mk;
    wl[wave][n] = l_run;
  }
  float* wacc_own = reinterpret_cast<float*>(&stage[wave][0]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float lo = __shfl_xor(acc[r][i], 32, 64);
      if (g < 2) wacc_own[(4 * g + i) * kD + 8 * n + r] = acc[r][i] + lo;
    }
  }
  __syncthreads();
  constexpr int nthr = kDecWaves * 64;
  float* part = a.part + ((size_t(unit) * a.nsplit + split) * kMaxHeads) * kPartStride;
  for (int e = tid; e < gc * kD; e += nthr) {
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
        A = fmaf(fw, reinterpret_cast<const float*>(&stage[w][0])[head * kD + dim], A);
      }
    }
    float* o = part + head * kPartStride;
    o[4 + dim] = A;
    if (dim == 0) {
      o[0] = M;
      o[1] = Ls;
    }
  }
}

// Lookup tables of the split kernel: value pairs (outlier codes in the lower
// half of rows 0..255, regular codes in the upper half of rows below
// kKeyRegRow), regular key pairs (rows kKeyRegRow + e, upper half) and
// outlier key pairs (rows kKeyOutRow + e for 3 bits; for 4 bits `tab2`, hi
// and lo pairs of copy c at 128e + 8c). Lane 16q + c of `cl` holds centroid c
// of codebook q: 0 outlier values, 1 regular values, 2 outlier keys, 3 regular
// keys. Stores and permutes as in build_tables.
template <int BK, int BV>
__device__ __forceinline__ void build_tables_o(float cl, float vsig, float ksig, uint8_t* tab, uint8_t* tab2,
                                               int tid, int nthr) {
  constexpr int BKO = BK + 1, BVO = BV + 1;
  constexpr int KVO = 1 << BVO, KV = 1 << BV;
  const uint32_t tb = lds_addr(tab);
  const float vs = kCentScale * vsig, ks = kCentScale * ksig;
  auto cent = [&](int q, int c, float sc) { return mul_rounded(lane_val(cl, 16 * q + c), sc); };
  for (int q = tid; q < 256 * 8; q += nthr) {
    const int e = q >> 3, c0 = e & 15, c1 = e >> 4;
    const uint32_t po = pack_h2(cent(0, c0 & (KVO - 1), vs), cent(0, c1 & (KVO - 1), vs));
    const uint32_t pr = pack_h2(cent(1, c0 & (KV - 1), vs), cent(1, c1 & (KV - 1), vs));
    const uint32_t wo = (c0 < KVO && c1 < KVO) ? po : 0u;
    lds_put4(tb + 256 * e + 16 * (q & 7), u32x4{wo, wo, wo, wo});
    if (e < kKeyRegRow) {
      const uint32_t wr = (c0 < KV && c1 < KV) ? pr : 0u;
      lds_put4(tb + 256 * e + kTabK + 16 * (q & 7), u32x4{wr, wr, wr, wr});
    }
  }
  constexpr int KR = 1 << (2 * BK);   // regular key pair entries
  // (whole wavefronts run the loop: the permutes in `cent` read every lane)
  constexpr int NQR = (KR * 8 + 63) / 64 * 64;
  for (int q = tid; q < NQR; q += nthr) {
    const int e = q >> 3;
    const uint32_t w = pack_h2(cent(3, e & ((1 << BK) - 1), ks), cent(3, (e >> BK) & ((1 << BK) - 1), ks));
    if (e < KR) lds_put4(tb + 256 * (kKeyRegRow + e) + kTabK + 16 * (q & 7), u32x4{w, w, w, w});
  }
  if constexpr (BKO == 4) {
    for (int q = tid; q < 256 * 8; q += nthr) {
      const int e = q >> 3;
      uint16_t h0, l0, h1, l1;
      split_h(cent(2, e & 15, ks), h0, l0);
      split_h(cent(2, e >> 4, ks), h1, l1);
      const uint32_t w0 = uint32_t(h0) | (uint32_t(h1) << 16), w1 = uint32_t(l0) | (uint32_t(l1) << 16);
      lds_put4(lds_addr(tab2) + 128 * e + 16 * (q & 7), u32x4{w0, w1, w0, w1});
    }
  } else {
    constexpr int KO = 1 << BKO;   // outlier key pair entries: e = code0 | code1 << BKO
    for (int q = tid; q < KO * KO * 8; q += nthr) {
      const int e = q >> 3;
      const uint32_t w = pack_h2(cent(2, e & (KO - 1), ks), cent(2, e >> BKO, ks));
      lds_put4(tb + 256 * (kKeyOutRow + e) + kTabK + 16 * (q & 7), u32x4{w, w, w, w});
    }
  }
}

template <int BK, int BV, bool AL, bool PROD>
__global__ __launch_bounds__(kDecWaves * 64) void attn_outlier_kernel(AttnArgs a) {
  using SL = OStage<BK, BV, PROD>;
  constexpr int BKO = BK + 1, BVO = BV + 1;
  __shared__ __attribute__((aligned(256))) uint8_t tab[kTabBytes];
  __shared__ __attribute__((aligned(256))) uint8_t tab2[BKO == 4 ? 256 * 128 : 16];
  __shared__ float wm[kDecWaves][kMaxHeads], wl[kDecWaves][kMaxHeads];
  __shared__ uint32_t prog[kDecWaves];   // blocks started per wavefront (issue balance)
  constexpr int kRing = kStages * SL::bytes > kMaxHeads * kD * 4 ? kStages * SL::bytes : kMaxHeads * kD * 4;
  __shared__ __attribute__((aligned(16))) uint8_t stage[kDecWaves][kRing];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int split = blockIdx.x, unit = blockIdx.y;
  const int grp = unit % a.ngroups;
  const int kvh = (unit / a.ngroups) % a.Hkv;
  const int b = unit / (a.ngroups * a.Hkv);
  const int gc = min(kMaxHeads, a.G - grp * kMaxHeads);
  constexpr int nthr = kDecWaves * 64;

  int64_t L = a.max_ctx;
  if (a.ctx_lens) {
    const int64_t l = a.ctx_lens[b];
    L = l < 0 ? 0 : (l > a.max_ctx ? a.max_ctx : l);
  }
  const int64_t per_wave = a.split_len / kDecWaves;
  const int64_t tb = int64_t(split) * a.split_len + wave * per_wave;
  const int64_t te = min(tb + per_wave, L);
  const uint32_t t_begin = static_cast<uint32_t>(tb);
  const uint32_t t_end = te > tb ? static_cast<uint32_t>(te) : t_begin;
  const uint32_t last = L > 0 ? static_cast<uint32_t>(L - 1) : 0u;
  const int64_t base = (int64_t(b) * a.Hkv + kvh) * a.max_ctx;
  const uint8_t* kc = a.kc + base * SL::KR;
  const uint8_t* vc = a.vc + base * SL::VR;
  const float* kn = a.kn + 2 * base;
  const float* vn = a.vn + 2 * base;
  const uint8_t* kqs = PROD ? a.kq + base * 16 : nullptr;
  const float* kgs = PROD ? a.kg + 2 * base : nullptr;

  // the four codebooks, the scales σ and the query operands go out before
  // the first blocks' loads (as in attn_split_kernel)
  float cl = 0.f;
  cl = codebook_group<1 << BVO>(a.vcent_o, 0, lane, cl);
  cl = codebook_group<1 << BV>(a.vcent, 1, lane, cl);
  cl = codebook_group<1 << BKO>(a.kcent_o, 2, lane, cl);
  cl = codebook_group<1 << BK>(a.kcent, 3, lane, cl);
  const float vsig = scalar_load(&a.vh->sigma), ksig = scalar_load(&a.kh->sigma);
  const uint8_t* blk = a.ws + size_t(unit) * kUnitBytes;
  const u32x4* fr = reinterpret_cast<const u32x4*>(blk);
  u32x4 bqo[4], bqr[4];   // the query fragments split by slot: outlier | regular
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const u32x4 v = fr[s * 64 + lane];
    bqo[s] = u32x4{v[0], 0u, 0u, 0u};
    bqr[s] = u32x4{0u, v[1], v[2], v[3]};
  }
  // Prod keys: the query's sketch operand split by position. K index k of the
  // operand is sketch coordinate 32(k/32) + 4c + m with k mod 32 = 8m + c; an
  // outlier coordinate (mod 8 < 2) has c even and m < 2, i.e. k mod 32 even
  // and below 16: the even bytes of lane groups 0 and 2.
  i32x8 bso[2], bsr[2];
  int ssc0 = 127, ssc1 = 127;
  if constexpr (PROD) {
    const i32x8* sk = reinterpret_cast<const i32x8*>(blk + kSkOff);
    const int32_t mo = ((lane >> 4) & 1) ? 0 : 0x00FF00FF;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const i32x8 v = sk[h * 64 + lane];
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        bso[h][d] = v[d] & mo;
        bsr[h][d] = v[d] & ~mo;
      }
    }
    const int32_t* ss = reinterpret_cast<const int32_t*>(blk + kSkScaleOff);
    ssc0 = ss[lane] + 2;       // ×4: both groups' √(π/2)/d_g share the factor 128/32
    ssc1 = ss[64 + lane] + 2;
  }
  const float iqs = reinterpret_cast<const float*>(blk + kQFrags * 1024)[n & 7];
  asm volatile("" ::: "memory");
  uint8_t* ring = &stage[wave][0];
  const uint32_t ring_addr = lds_addr(ring);
  const OOffsets so = ostage_offsets<BK, BV>(n, g);
  const uint32_t nblk = (t_end - t_begin + kBlockTok - 1) / kBlockTok;
  auto stage_at = [&](uint8_t* st, uint32_t t0) {
    ostage_block<BK, BV, AL, PROD>(st, t0, last, lane, kc, vc, kn, vn, kqs, kgs);
  };
  if (nblk > 0) stage_at(ring, t_begin);
  if (nblk > 1) stage_at(ring + SL::bytes, t_begin + kBlockTok);

  build_tables_o<BK, BV>(cl, vsig, ksig, tab, tab2, tid, nthr);
  if (tid < kDecWaves) lds_put1(lds_addr(&prog[tid]), 0u);
  lds_stores_done();
  const uint32_t cp = lane & 31;
  const uint32_t lane_lo = 4u * cp, lane_hi = kTabK + 4u * cp, lane8 = 8u * (lane & 15);
  const bool own1 = n >= 8;                 // the lane's own tile: tokens 16..31 of each block
  const uint32_t own_off = own1 ? 128u : 0u;
  tables_barrier();

  SoftmaxState st{-INFINITY, -INFINITY, 0.f, 0.f, 0.f, INFINITY};
  f32x4 acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
  // issue balance between the two wavefronts of a SIMD, as in attn_split_kernel
  const uint32_t prog_own = lds_addr(&prog[wave]), prog_partner = lds_addr(&prog[wave ^ 4]);
  int cur = 0;
  for (uint32_t i = 0; i < nblk; ++i) {
    const uint32_t t0 = t_begin + i * kBlockTok;
    OBlock R;
    const uint32_t sb = ring_addr + cur * SL::bytes;
    lds_put1(prog_own, i);
    uint32_t pw;
    if (i + 1 < nblk)
      oread_block<BK, BV, SL::dma>(R, sb, so, own_off, prog_partner, pw);
    else
      oread_block<BK, BV, 0>(R, sb, so, own_off, prog_partner, pw);
    if constexpr (PROD) oread_prod<BK, BV>(R, sb, n, g);
    if (__builtin_amdgcn_readfirstlane(pw) < i)
      __builtin_amdgcn_s_setprio(0);
    else
      __builtin_amdgcn_s_setprio(1);
    if (i + 2 < nblk) {
      const int nx = (cur + 2) % kStages;
      stage_at(ring + nx * SL::bytes, t0 + 2 * kBlockTok);
    }
    oattend_block<BK, BV, PROD>(R, t0, t_end, n, g, tab, tab2, lane_lo, lane_hi, lane8, bqo, bqr, bso, bsr, ssc0,
                                ssc1, iqs, own1, st, acc);
    cur = cur + 1 == kStages ? 0 : cur + 1;
  }
  __builtin_amdgcn_s_setprio(0);
  write_partials_o<kRing>(a, st, acc, wm, wl, stage, unit, split, gc, n, g, wave, tid);
}

template <int BK, int BV, bool PROD = false>
hipError_t launch_outlier_t(const AttnArgs& a, bool al, dim3 grid, hipStream_t st) {
  if (al)
    hipLaunchKernelGGL((attn_outlier_kernel<BK, BV, true, PROD>), grid, dim3(kDecWaves * 64), 0, st, a);
  else
    hipLaunchKernelGGL((attn_outlier_kernel<BK, BV, false, PROD>), grid, dim3(kDecWaves * 64), 0, st, a);
  return hipGetLastError();
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

// One workgroup per unit. Log-sum-exp combination of the splits per (head,
// dim), then o = Π_Vᵀ·acc for the unit's heads: thread t takes output dim
// t % 128 over a quarter of the contraction, so each row of Π_V is read once
// for all heads. All loads of a thread are issued before their first use
// (the Π_V column piece, then up to 16 splits' partials at a time).
constexpr int kMergeChunk = 16;

__global__ __launch_bounds__(kD) void merge_kernel(MergeArgs a) {
  // One workgroup per (unit, head); thread d owns output dim d. Every load
  // (the column of Π_V, then the splits' partials) is issued before the
  // first use, so the launch costs about one memory round trip.
  __shared__ float accs[kD];
  const int unit = blockIdx.x / kMaxHeads, head = blockIdx.x % kMaxHeads;
  const int grp = unit % a.ngroups;
  const int kvh = (unit / a.ngroups) % a.Hkv;
  const int b = unit / (a.ngroups * a.Hkv);
  const int gc = min(kMaxHeads, a.G - grp * kMaxHeads);
  if (head >= gc) return;   // uniform over the workgroup
  const int d = threadIdx.x;
  float pv[kD];             // Π_V[k][d]: o_d = Σ_k Π_V[k][d]·acc_k
#pragma unroll
  for (int k = 0; k < kD; ++k) pv[k] = a.rot_v[k * kD + d];
  const float* ph = a.part + (size_t(unit) * a.nsplit * kMaxHeads + head) * kPartStride;
  const size_t sstride = size_t(kMaxHeads) * kPartStride;
  const float inv_cs = 1.0f / (kCentScale * a.vh->sigma);
  float M = -INFINITY, Ls = 0.f, A = 0.f;
  for (int s0 = 0; s0 < a.nsplit; s0 += kMergeChunk) {
    // unconditional loads (clamped to the last split), masked at use
    float ms[kMergeChunk], ls[kMergeChunk], as[kMergeChunk];
#pragma unroll
    for (int i = 0; i < kMergeChunk; ++i) {
      const float* q = ph + size_t(min(s0 + i, a.nsplit - 1)) * sstride;
      ms[i] = q[0];
      ls[i] = q[1];
      as[i] = q[4 + d];
    }
    float mc = M;
#pragma unroll
    for (int i = 0; i < kMergeChunk; ++i) {
      if (s0 + i >= a.nsplit) ms[i] = -INFINITY;
      mc = fmaxf(mc, ms[i]);
    }
    if (mc > -INFINITY) {
      const float fo = M > -INFINITY ? exp2f(M - mc) : 0.f;
      Ls *= fo;
      A *= fo;
#pragma unroll
      for (int i = 0; i < kMergeChunk; ++i) {
        const float fw = s0 + i < a.nsplit ? exp2f(ms[i] - mc) : 0.f;
        Ls = fmaf(fw, ls[i], Ls);
        A = fmaf(fw, as[i], A);
      }
      M = mc;
    }
  }
  accs[d] = Ls > 0.f ? A * inv_cs / Ls : 0.f;
  __syncthreads();
  float o = 0.f;
#pragma unroll
  for (int k = 0; k < kD; ++k) o = fmaf(pv[k], accs[k], o);
  const size_t hq = size_t(b) * a.Hq + kvh * a.G + grp * kMaxHeads + head;
  a.out[hq * kD + d] = o;
}

// ---------------------------------------------------------------------------
// 4. Inner-product search over a packed database
// ---------------------------------------------------------------------------
// The k database vectors with the largest ⟨q, x̃⟩ for each query ("内存厂商的
// 噩梦来了…" (wuyi.wiki) section 6.4: nearest-neighbour search by inner product
// over TurboQuant-encoded vectors). The scores are the decode kernel's key
// scores with the softmax scale chosen so that they are plain inner
// products: query operands from query_prep_kernel for groups of up to 8
// queries, then one workgroup per (split, query group) streams its share of
// the database through the decode kernel's LDS staging and tables, keys only.
//
// A candidate (score, index) is better than another when its score is larger,
// or equal with a smaller index. As one 64-bit key: the score's
// order-preserving bits above the complement of the index; 0 is below every
// candidate.
constexpr int kSearchMaxK = 32;
constexpr int kCand = 64;          // candidate slots per (wavefront, query)

__device__ __forceinline__ uint64_t cand_key(float s, uint32_t idx) {
  const uint32_t b = __builtin_bit_cast(uint32_t, s + 0.0f);   // -0 ranks as +0
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (uint64_t(o) << 32) | uint64_t(~idx);
}
__device__ __forceinline__ float key_score(uint64_t k) {
  const uint32_t o = uint32_t(k >> 32);
  return __builtin_bit_cast(float, (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ uint32_t key_index(uint64_t k) { return ~uint32_t(k); }

// Value of lane (lane ^ M) of v for M = 1, 2, 4, 8, 16, 32: DPP moves within
// rows (quad permutes; a half-row mirror, i ^ 7, then the quad reversal,
// i ^ 3; a rotation by 8) and the gfx950 row swaps across rows, none of which
// goes through the LDS pipe as a general lane shuffle does.
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v, int lane) {
  if constexpr (M == 1) {
    return __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, false);          // quad_perm 1,0,3,2
  } else if constexpr (M == 2) {
    return __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false);          // quad_perm 2,3,0,1
  } else if constexpr (M == 4) {
    const uint32_t m = __builtin_amdgcn_update_dpp(0u, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    return __builtin_amdgcn_update_dpp(0u, m, 0x1B, 0xF, 0xF, false);          // quad_perm 3,2,1,0
  } else if constexpr (M == 8) {
    return __builtin_amdgcn_update_dpp(0u, v, 0x128, 0xF, 0xF, false);         // row_ror 8
  } else if constexpr (M == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16) ? p[0] : p[1];
  } else {
    static_assert(M == 32, "xor_lane");
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane & 32) ? p[0] : p[1];
  }
}
template <int M>
__device__ __forceinline__ uint64_t xor_lane64(uint64_t v, int lane) {
  return (uint64_t(xor_lane<M>(uint32_t(v >> 32), lane)) << 32) | xor_lane<M>(uint32_t(v), lane);
}
// Value of lane 63 - lane: the row mirror (i ^ 15), then across rows.
__device__ __forceinline__ uint64_t reverse_lanes64(uint64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, uint32_t(v), 0x140, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, uint32_t(v >> 32), 0x140, 0xF, 0xF, false);
  return xor_lane64<32>(xor_lane64<16>((uint64_t(hi) << 32) | lo, lane), lane);
}

// Compare-exchange steps STRIDE, STRIDE/2, ..., 1 of a bitonic network whose
// blocks of SIZE lanes alternate direction (SIZE = 64: one descending run); in
// a pair, the lower lane of a descending block keeps the larger key.
template <int SIZE, int STRIDE>
__device__ __forceinline__ uint64_t bitonic_steps(uint64_t k, int lane) {
  const uint64_t p = xor_lane64<STRIDE>(k, lane);
  const bool keep_max = ((lane & SIZE) == 0) == ((lane & STRIDE) == 0);
  k = keep_max ? (k > p ? k : p) : (k < p ? k : p);
  if constexpr (STRIDE > 1)
    return bitonic_steps<SIZE, STRIDE / 2>(k, lane);
  else
    return k;
}
template <int SIZE>
__device__ __forceinline__ uint64_t bitonic_sort_from(uint64_t k, int lane) {
  k = bitonic_steps<SIZE, SIZE / 2>(k, lane);
  if constexpr (SIZE < 64)
    return bitonic_sort_from<SIZE * 2>(k, lane);
  else
    return k;
}

// Bitonic sort of one key per lane over the 64 lanes, best (largest) first.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t k, int lane) { return bitonic_sort_from<2>(k, lane); }

// Merge of a bitonic sequence over the 64 lanes (lanes 0..31 descending,
// lanes 32..63 ascending) into one descending run: two sorted lists of up to
// 32 keys, the second loaded in reverse order, in six compare-exchange steps.
__device__ __forceinline__ uint64_t wave_merge_desc(uint64_t k, int lane) { return bitonic_steps<64, 32>(k, lane); }

// Candidate buffers of a search workgroup: per (wavefront, query) up to kCand
// keys, and the count each wavefront holds at the end of its scan.
struct SearchLds {
  uint64_t cand[kDecWaves][kMaxHeads][kCand];
  uint32_t cnt[kDecWaves][kMaxHeads];
};

// A candidate store the compiler does not see as an LDS access: as a plain
// store it would first wait for every direct-to-LDS load in flight (it cannot
// tell the candidate buffer from the staging ring), which stalls the scan on
// the prefetch of the block after next. A wavefront's LDS accesses execute in
// order, so the compaction's reads still see these stores.
__device__ __forceinline__ void lds_store_key(uint32_t addr, uint64_t v) {
  asm volatile("ds_write_b64 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// Sort the m (<= kCand) candidates of query c, keep the best k (best first)
// and return the k-th score, the bar for new candidates (-inf while fewer
// than k are held). Whole wavefront.
__device__ __forceinline__ float compact_cands(SearchLds& S, int wave, int c, int k, int lane, uint32_t m) {
  uint64_t key = uint32_t(lane) < m ? S.cand[wave][c][lane] : 0ull;
  key = wave_sort_desc(key, lane);
  if (lane < k) S.cand[wave][c][lane] = key;
  const uint32_t klo = __builtin_amdgcn_readlane(uint32_t(key), k - 1);
  const uint32_t khi = __builtin_amdgcn_readlane(uint32_t(key >> 32), k - 1);
  return m >= uint32_t(k) ? key_score((uint64_t(khi) << 32) | klo) : -INFINITY;
}

struct SearchArgs {
  const uint8_t* kc;
  const float* kn;
  const uint8_t* kq;
  const float* kg;
  int64_t n;
  const float* kcent;
  const PrepHeader* kh;
  const uint8_t* ws;
  uint64_t* part;     // [units][nsplit][8][k] best-first keys of each split
  int ngroups, nq, nsplit, split_len, k;
  // Chunked vectors (one pass per 128-coordinate chunk): partial[q·n + v] holds
  // query q's summed score of vector v over the chunks before this pass.
  float* partial;
  int pin;            // add partial to this pass's scores
  int pout;           // store the sums to partial and keep no candidates
};

// LDS of the search scan: the key table holds only the rows its entries use
// (no value half), and the rest of the 160 KiB goes to a deeper staging ring
// than the decode kernel's, since a keys-only block carries half the bytes.
template <int BK, bool PROD>
struct SearchPlan {
  using KL = KLut<BK>;
  static constexpr int tab_bytes = KL::priv ? KL::entries * 256 : 256;
  static constexpr int fixed = tab_bytes + KL::bytes + int(sizeof(SearchLds)) + 64 + 1024;
  static constexpr int ring = (160 * 1024 - fixed) / (kDecWaves * Stage<BK, PROD, 0>::bytes);
  static constexpr int stages = ring > 4 ? 4 : ring;
  static_assert(stages >= 2, "search staging ring");
};

template <int BK, bool PROD, bool AL>
__global__ __launch_bounds__(kDecWaves * 64) void search_scan_kernel(SearchArgs a) {
  using SL = Stage<BK, PROD, 0>;
  using KL = KLut<BK>;
  constexpr int NST = SearchPlan<BK, PROD>::stages;
  __shared__ __attribute__((aligned(256))) uint8_t tab[SearchPlan<BK, PROD>::tab_bytes];
  __shared__ __attribute__((aligned(16))) uint8_t lut_k[KL::bytes];
  __shared__ __attribute__((aligned(16))) uint8_t stage[kDecWaves][NST * SL::bytes];
  __shared__ SearchLds S;
  __shared__ uint32_t prog[kDecWaves];   // blocks started per wavefront (issue balance)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int split = blockIdx.x, unit = blockIdx.y;
  const int gc = min(kMaxHeads, a.nq - unit * kMaxHeads);
  const int k = a.k;
  constexpr int nthr = kDecWaves * 64;

  // ---- token range of this wavefront ----
  const int64_t per_wave = a.split_len / kDecWaves;
  const int64_t tb = int64_t(split) * a.split_len + wave * per_wave;
  const int64_t te = min(tb + per_wave, a.n);
  const uint32_t t_begin = static_cast<uint32_t>(tb);
  const uint32_t t_end = te > tb ? static_cast<uint32_t>(te) : t_begin;
  const uint32_t last = static_cast<uint32_t>(a.n - 1);
  const uint8_t* kc = BK > 0 ? a.kc : reinterpret_cast<const uint8_t*>(a.kn);
  const uint8_t* kq = PROD ? a.kq : reinterpret_cast<const uint8_t*>(a.kn);
  const float* kg = PROD ? a.kg : a.kn;

  // ---- codebook, scale and query operands, then the first blocks' loads
  // (as in attn_split_kernel) ----
  constexpr int KK = BK > 0 ? (1 << BK) : 1;
  const float kcl = BK > 0 ? codebook_lanes<KK>(a.kcent, n) : 0.f;
  const float ksig = BK > 0 ? scalar_load(&a.kh->sigma) : 0.f;
  const uint8_t* blk = a.ws + size_t(unit) * kUnitBytes;
  const u32x4* fr = reinterpret_cast<const u32x4*>(blk);
  u32x4 bq[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) bq[s] = fr[s * 64 + lane];
  i32x8 bs[2];
  int ssc0 = 127, ssc1 = 127;
  if constexpr (PROD) {
    const i32x8* sk = reinterpret_cast<const i32x8*>(blk + kSkOff);
    bs[0] = sk[lane];
    bs[1] = sk[64 + lane];
    const int32_t* ss = reinterpret_cast<const int32_t*>(blk + kSkScaleOff);
    ssc0 = ss[lane];
    ssc1 = ss[64 + lane];
  }
  const float iqs = reinterpret_cast<const float*>(blk + kQFrags * 1024)[n & 7];
  asm volatile("" ::: "memory");
  uint8_t* ring = &stage[wave][0];
  const uint32_t ring_addr = lds_addr(ring);
  const StageOffsets so = stage_offsets<BK, PROD, 0>(n, g);
  const DmaLane dl = dma_lane<BK, 0>(lane);
  const uint32_t nblk = (t_end - t_begin + kBlockTok - 1) / kBlockTok;
#pragma unroll
  for (int b = 0; b < NST; ++b)
    if (uint32_t(b) < nblk)
      stage_block<BK, PROD, 0, AL>(ring + b * SL::bytes, t_begin + b * kBlockTok, last, lane, dl, kc, kq, kc, a.kn,
                                   a.kn, kg);

  // ---- key tables (as in the decode kernel, no value table) ----
  build_tables<BK, 0>(0.f, kcl, 0.f, ksig, tab, lut_k, tid, nthr);
  if (tid < kDecWaves) lds_put1(lds_addr(&prog[tid]), 0u);
  lds_stores_done();
  Luts T;
  const uint32_t cp = lane & 31;
  T.k = KL::priv ? tab : lut_k;
  T.v = tab;
  T.klane = KL::byte_indexed ? kTabK + 8u * (lane & 15) : KL::priv ? kTabK + 4u * cp : 0u;
  T.vlane = 4u * cp;
  tables_barrier();

  // ---- scan: scores of 32 vectors per block; candidates above the bar go to
  // the buffer of their query. Lanes n and n + 8 hold query n % 8 with equal
  // scores and keep equal counts; lanes n < 8 store. ----
  const int c = n & 7;
  const bool live = c < gc;
  const uint32_t cand_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&S.cand[wave][c][0]));
  float bar = -INFINITY;
  uint32_t cnt = 0;
  int cur = 0;
  const uint32_t prog_own = lds_addr(&prog[wave]), prog_partner = lds_addr(&prog[wave ^ 4]);
  for (uint32_t i = 0; i < nblk; ++i) {
    const uint32_t t0 = t_begin + i * kBlockTok;
    Block<BK, PROD, 0> R;
    const uint32_t sb = ring_addr + cur * SL::bytes;
    // the blocks after this one already issued: their loads may stay in flight
    const uint32_t ahead = min(nblk - 1 - i, uint32_t(NST - 1));
    // issue balance between the two wavefronts of a SIMD, as in attn_split_kernel
    lds_put1(prog_own, i);
    uint32_t pw;
    if (ahead == uint32_t(NST - 1))
      read_block<BK, PROD, 0, (NST - 1) * SL::dma>(R, sb, so, prog_partner, pw);
    else if (NST > 3 && ahead == 2)
      read_block<BK, PROD, 0, (NST > 3 ? 2 : 0) * SL::dma>(R, sb, so, prog_partner, pw);
    else if (NST > 2 && ahead == 1)
      read_block<BK, PROD, 0, (NST > 2 ? 1 : 0) * SL::dma>(R, sb, so, prog_partner, pw);
    else
      read_block<BK, PROD, 0, 0>(R, sb, so, prog_partner, pw);
    if (__builtin_amdgcn_readfirstlane(pw) < i)
      __builtin_amdgcn_s_setprio(0);
    else
      __builtin_amdgcn_s_setprio(1);
    if (i + NST < nblk)
      stage_block<BK, PROD, 0, AL>(ring + cur * SL::bytes, t0 + NST * kBlockTok, last, lane, dl, kc, kq, kc, a.kn,
                                   a.kn, kg);
    float sc[8];
    block_scores<BK, PROD, 0>(R, T, bq, bs, ssc0, ssc1, sc);
#pragma unroll
    for (int j = 0; j < 8; ++j) sc[j] *= iqs;
    if (a.pin | a.pout) {
      // chunked vectors: the sum over this and the earlier chunks' passes
      // (lanes n and n + 8 hold the same scores; lanes n < 8 load and store)
      float* pq = a.partial + size_t(unit * kMaxHeads + c) * size_t(a.n);
      const bool io = live && n < 8;
      if (a.pin) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t t = t0 + 16 * (j >> 2) + 4 * g + (j & 3);
          sc[j] += (io && t < t_end) ? pq[t] : 0.f;
        }
      }
      if (a.pout) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t t = t0 + 16 * (j >> 2) + 4 * g + (j & 3);
          if (io && t < t_end) pq[t] = sc[j];
        }
        cur = cur + 1 == NST ? 0 : cur + 1;
        continue;
      }
    }
    uint32_t msk = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t t = t0 + 16 * (j >> 2) + 4 * g + (j & 3);
      if (t < t_end && sc[j] > bar) msk |= 1u << j;
    }
    if (!live) msk = 0;
    // slots of this lane's candidates: after those of the lower lane groups
    // (lanes n + 16g, g = 0..3, hold the same query)
    const uint32_t nl = __builtin_popcount(msk);
    const uint32_t n16 = xor_lane<16>(nl, lane);
    const uint32_t pair = nl + n16;
    const uint32_t p32 = xor_lane<32>(pair, lane);
    const uint32_t total = pair + p32;
    // one candidate per lane per round, lowest slot first (usually one round)
    uint32_t rem = n < 8 ? msk : 0u;
    uint32_t pos = cnt + ((g & 1) ? n16 : 0u) + ((g & 2) ? p32 : 0u);
    while (__ballot(rem != 0u)) {
      if (rem != 0u) {
        const uint32_t j = __builtin_ctz(rem);
        rem &= rem - 1u;
        const bool b0 = j & 1u, b1 = j & 2u, b2 = j & 4u;
        const float a0 = b0 ? sc[1] : sc[0], a1 = b0 ? sc[3] : sc[2];
        const float a2 = b0 ? sc[5] : sc[4], a3 = b0 ? sc[7] : sc[6];
        const float s = b2 ? (b1 ? a3 : a2) : (b1 ? a1 : a0);
        const uint32_t t = t0 + 16 * (j >> 2) + 4 * g + (j & 3);
        if (pos < uint32_t(kCand)) lds_store_key(cand_base + 8 * pos, cand_key(s, t));
        ++pos;
      }
    }
    cnt += total;
    // at most 32 new candidates per query per block: keep the best k of a
    // query once it holds more than 32
    uint64_t over = __ballot(lane < kMaxHeads && cnt > uint32_t(kCand / 2));
    while (over) {
      const int q = __builtin_ctzll(over);
      over &= over - 1;
      const uint32_t mq = __builtin_amdgcn_readlane(cnt, q);
      const float thr = compact_cands(S, wave, q, k, lane, mq);
      if (c == q) {
        cnt = mq < uint32_t(k) ? mq : uint32_t(k);
        bar = thr;
      }
    }
    cur = cur + 1 == NST ? 0 : cur + 1;
  }
  __builtin_amdgcn_s_setprio(0);
  for (int q = 0; q < gc; ++q) {
    const uint32_t mq = __builtin_amdgcn_readlane(cnt, q);
    compact_cands(S, wave, q, k, lane, mq);
    if (lane == 0) S.cnt[wave][q] = mq < uint32_t(k) ? mq : uint32_t(k);
  }
  __syncthreads();

  // ---- the workgroup's best k per query: wavefront q merges query q's lists
  // (each sorted, best first) ----
  if (wave < gc) {
    const int q = wave;
    uint64_t best = 0ull;
    for (int w = 0; w < kDecWaves; ++w) {
      const uint32_t m = S.cnt[w][q];
      uint64_t key = best;
      if (lane >= 32) key = uint32_t(63 - lane) < m ? S.cand[w][q][63 - lane] : 0ull;
      best = wave_merge_desc(key, lane);
    }
    if (lane < k) a.part[((size_t(unit) * a.nsplit + split) * kMaxHeads + q) * a.k + lane] = best;
  }
}

// The 32 best of two descending runs of a wavefront's lanes 0..31: a in this
// call's lanes 0..31, b's lanes 0..31 reversed into lanes 32..63.
__device__ __forceinline__ uint64_t merge_runs(uint64_t a, uint64_t b, int lane) {
  const uint64_t r = reverse_lanes64(b, lane);
  return wave_merge_desc(lane < 32 ? a : r, lane);
}

// One workgroup per query: the best k over all splits, best first.
// Wavefront w runs kMergeChains independent merge chains over splits
// w + 8c + 8·kMergeChains·r (round r), with round r + 1's lists loaded before
// round r merges; the chains then merge within the wavefront and the
// wavefronts' runs in a three-level tree.
constexpr int kMergeChains = 4;
__global__ __launch_bounds__(kDecWaves * 64) void search_merge_kernel(const uint64_t* __restrict__ part, int nsplit,
                                                                      int k, float* __restrict__ scores,
                                                                      int64_t* __restrict__ index) {
  __shared__ uint64_t wbest[kDecWaves][32];
  const int qi = blockIdx.x;
  const int unit = qi / kMaxHeads, q = qi % kMaxHeads;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const uint64_t* lists = part + size_t(unit) * nsplit * kMaxHeads * k;
  // lanes 32..63 hold a list reversed (lane 63 its best), the rest 0. Every
  // lane loads from an address inside the lists and the keys it does not hold
  // are cleared only when merged, so no load sits under a branch and the next
  // round's loads stay in flight while this round merges.
  const bool upper = lane >= 32 && 63 - lane < k;
  const int ek = min(63 - lane, k - 1);
  auto list_key = [&](int s) -> uint64_t {
    return lists[(size_t(min(s, nsplit - 1)) * kMaxHeads + q) * k + ek];
  };
  constexpr int step = kDecWaves * kMergeChains;
  uint64_t best[kMergeChains], nxt[kMergeChains];
#pragma unroll
  for (int c = 0; c < kMergeChains; ++c) {
    best[c] = 0ull;
    nxt[c] = list_key(wave + kDecWaves * c);
  }
  for (int s0 = wave; s0 < nsplit; s0 += step) {
    uint64_t cur[kMergeChains];
#pragma unroll
    for (int c = 0; c < kMergeChains; ++c) {
      cur[c] = nxt[c];
      nxt[c] = list_key(s0 + step + kDecWaves * c);
    }
#pragma unroll
    for (int c = 0; c < kMergeChains; ++c) {
      const uint64_t x = (upper && s0 + kDecWaves * c < nsplit) ? cur[c] : 0ull;
      best[c] = wave_merge_desc(lane < 32 ? best[c] : x, lane);
    }
  }
  uint64_t b = merge_runs(merge_runs(best[0], best[1], lane), merge_runs(best[2], best[3], lane), lane);
  if (lane < 32) wbest[wave][lane] = b;
  __syncthreads();
#pragma unroll
  for (int span = 1; span < kDecWaves; span *= 2) {
    if ((wave & (2 * span - 1)) == 0) {
      const uint64_t o = lane >= 32 ? wbest[wave + span][63 - lane] : 0ull;
      b = wave_merge_desc(lane < 32 ? b : o, lane);
    }
    __syncthreads();
    if ((wave & (2 * span - 1)) == 0 && lane < 32) wbest[wave][lane] = b;
    __syncthreads();
  }
  if (wave == 0 && lane < k) {
    scores[size_t(qi) * k + lane] = key_score(b);
    index[size_t(qi) * k + lane] = static_cast<int64_t>(key_index(b));
  }
}

template <int BK, bool PROD>
hipError_t launch_search_t(const SearchArgs& a, bool al, dim3 grid, hipStream_t st) {
  if (al)
    hipLaunchKernelGGL((search_scan_kernel<BK, PROD, true>), grid, dim3(kDecWaves * 64), 0, st, a);
  else
    hipLaunchKernelGGL((search_scan_kernel<BK, PROD, false>), grid, dim3(kDecWaves * 64), 0, st, a);
  return hipGetLastError();
}

template <int BK, bool PROD, int BV>
hipError_t launch_attn_t(const AttnArgs& a, bool al, dim3 grid, hipStream_t st) {
  if (al)
    hipLaunchKernelGGL((attn_split_kernel<BK, PROD, BV, true>), grid, dim3(kDecWaves * 64), 0, st, a);
  else
    hipLaunchKernelGGL((attn_split_kernel<BK, PROD, BV, false>), grid, dim3(kDecWaves * 64), 0, st, a);
  return hipGetLastError();
}

template <int BK, bool PROD>
hipError_t launch_attn_bv(const AttnArgs& a, int bv, bool al, dim3 grid, hipStream_t st) {
  switch (bv) {
    case 1: return launch_attn_t<BK, PROD, 1>(a, al, grid, st);
    case 2: return launch_attn_t<BK, PROD, 2>(a, al, grid, st);
    case 3: return launch_attn_t<BK, PROD, 3>(a, al, grid, st);
    default: return launch_attn_t<BK, PROD, 4>(a, al, grid, st);
  }
}


}  // namespace tq

using namespace tq;

extern "C" size_t tq_attn_decode_workspace(int B, int Hq, int Hkv, int64_t max_ctx) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_ctx < 1 || max_ctx > kMaxCtx) return 0;
  return make_plan(B, Hq, Hkv, max_ctx).bytes;
}

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The new key and value rows of a decode step (null for plain decode).
struct StepRows {
  const void* k_new;
  const void* v_new;
  int x_dtype;
  int64_t x_row_stride;
};

RowEncArgs append_args(const tq_quantizer* q, const StepRows& r, const void* x, int rows, const int32_t* ctx_lens,
                       int64_t max_ctx, int Hkv, const tq_packed* cache) {
  RowEncArgs e{};
  const bool prod = q->variant == TQ_PROD;
  e.x = x;
  e.n = rows;
  e.stride = r.x_row_stride;
  e.f32in = r.x_dtype == TQ_F32;
  e.bm = prod ? q->bits - 1 : q->bits;
  e.prod = prod;
  e.codes = cache->codes;
  e.norms = cache->norms;
  e.qjl = cache->qjl;
  e.gammas = cache->gammas;
  e.frags = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(q->prep) + kPrepHeaderBytes);
  e.centroids = q->centroids;
  e.boundaries = q->boundaries;
  e.slot = nullptr;
  e.lens = ctx_lens;
  e.max_ctx = max_ctx;
  e.hkv = Hkv;
  e.append = 1;
  return e;
}

int decode_call(int phase, const tq_quantizer* kq, const tq_quantizer* vq, const float* query, int B,
                int Hq, int Hkv, const int32_t* ctx_lens, int64_t max_ctx, const tq_packed* k_cache,
                const tq_packed* v_cache, float scale, float* out, void* workspace, size_t ws_bytes,
                void* stream, const StepRows* step = nullptr, bool checks_only = false) {
  if (phase < 0 || phase > 3) return TQ_ERR_INVALID_ARG;
  int st = tq_check_quantizer(kq);
  if (st != TQ_OK) return st;
  st = tq_check_quantizer(vq);
  if (st != TQ_OK) return st;
  if (vq->variant != TQ_MSE) return TQ_ERR_UNSUPPORTED;
  // Split caches: both quantizers split.
  const bool osplit = kq->split != TQ_SPLIT_NONE;
  if (osplit != (vq->split != TQ_SPLIT_NONE)) return TQ_ERR_UNSUPPORTED;
  if (query == nullptr || out == nullptr || k_cache == nullptr || v_cache == nullptr || workspace == nullptr)
    return TQ_ERR_INVALID_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_ctx < 1) return TQ_ERR_INVALID_ARG;
  if (max_ctx > kMaxCtx) return TQ_ERR_UNSUPPORTED;
  const bool prod = kq->variant == TQ_PROD;
  const int bk = prod ? kq->bits - 1 : kq->bits;
  if (k_cache->norms == nullptr || (bk > 0 && k_cache->codes == nullptr)) return TQ_ERR_INVALID_ARG;
  if (prod && (k_cache->qjl == nullptr || k_cache->gammas == nullptr)) return TQ_ERR_INVALID_ARG;
  if (v_cache->norms == nullptr || v_cache->codes == nullptr) return TQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(k_cache->codes) | reinterpret_cast<uintptr_t>(v_cache->codes) |
       reinterpret_cast<uintptr_t>(prod ? k_cache->qjl : nullptr)) % 16 != 0)
    return TQ_ERR_INVALID_ARG;
  if (step != nullptr) {
    // The appended rows are written through the same pointers.
    if (step->x_dtype != TQ_F32 && step->x_dtype != TQ_BF16) return TQ_ERR_UNSUPPORTED;
    if (step->k_new == nullptr || step->v_new == nullptr || !aligned(step->k_new, 16) ||
        !aligned(step->v_new, 16) || step->x_row_stride < TQ_HEAD_DIM || step->x_row_stride % 8 != 0)
      return TQ_ERR_INVALID_ARG;
    if (!aligned(k_cache->norms, 4) || !aligned(v_cache->norms, 4) || (prod && !aligned(k_cache->gammas, 4)))
      return TQ_ERR_INVALID_ARG;
    if (int64_t(B) * Hkv > (int64_t(1) << 30)) return TQ_ERR_UNSUPPORTED;
  }
  const Plan p = make_plan(B, Hq, Hkv, max_ctx);
  if (ws_bytes < p.bytes || reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return TQ_ERR_WORKSPACE;
  if (checks_only) return TQ_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const int G = Hq / Hkv;
  float* part = reinterpret_cast<float*>(ws + p.part_off);

  if (phase == 0 || phase == 1) {
    PrepArgs pa{query, tq_rotation_matrix(kq), tq_projection_matrix(kq), static_cast<const PrepHeader*>(kq->prep), scale,
                Hq, Hkv, G, p.ngroups, p.units, ws};
    if (step == nullptr) {
      hipLaunchKernelGGL(query_prep_kernel, dim3(p.units), dim3(kRowWaves * 64), 0, s, pa);
    } else if (osplit) {
      // split caches: the query operands, then the split encoder's appends
      // of the keys and the values (three launches)
      hipLaunchKernelGGL(query_prep_kernel, dim3(p.units), dim3(kRowWaves * 64), 0, s, pa);
      if (hipGetLastError() != hipSuccess) return TQ_ERR_HIP;
      const int rows = B * Hkv;
      st = tq_split_append(kq, step->k_new, step->x_dtype, rows, step->x_row_stride, k_cache, ctx_lens, max_ctx,
                           Hkv, stream);
      if (st != TQ_OK) return st;
      st = tq_split_append(vq, step->v_new, step->x_dtype, rows, step->x_row_stride, v_cache, ctx_lens, max_ctx,
                           Hkv, stream);
      if (st != TQ_OK) return st;
    } else {
      StepArgs sa;
      sa.prep = pa;
      const int rows = B * Hkv;
      sa.kenc = append_args(kq, *step, step->k_new, rows, ctx_lens, max_ctx, Hkv, k_cache);
      sa.venc = append_args(vq, *step, step->v_new, rows, ctx_lens, max_ctx, Hkv, v_cache);
      sa.ktiles = sa.vtiles = (rows + 15) / 16;
      hipLaunchKernelGGL(step_prologue_kernel, dim3(sa.ktiles + sa.vtiles + p.units), dim3(kRowWaves * 64), 0, s, sa);
    }
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
    aa.kcent_o = kq->centroids_o;
    aa.vcent_o = vq->centroids_o;
    const dim3 grid(p.nsplit, p.units);
    const int bv = vq->bits;
    const bool al = (max_ctx % kBlockTok) == 0;
    hipError_t e;
    if (osplit && prod) {
      // prod keys: regular Lloyd-Max width bits - 1 (1 or 2)
      if (bk == 1)
        e = bv == 2 ? launch_outlier_t<1, 2, true>(aa, al, grid, s) : launch_outlier_t<1, 3, true>(aa, al, grid, s);
      else
        e = bv == 2 ? launch_outlier_t<2, 2, true>(aa, al, grid, s) : launch_outlier_t<2, 3, true>(aa, al, grid, s);
    } else if (osplit) {
      if (bk == 2)
        e = bv == 2 ? launch_outlier_t<2, 2>(aa, al, grid, s) : launch_outlier_t<2, 3>(aa, al, grid, s);
      else
        e = bv == 2 ? launch_outlier_t<3, 2>(aa, al, grid, s) : launch_outlier_t<3, 3>(aa, al, grid, s);
    } else if (!prod) {
      switch (bk) {
        case 1: e = launch_attn_bv<1, false>(aa, bv, al, grid, s); break;
        case 2: e = launch_attn_bv<2, false>(aa, bv, al, grid, s); break;
        case 3: e = launch_attn_bv<3, false>(aa, bv, al, grid, s); break;
        default: e = launch_attn_bv<4, false>(aa, bv, al, grid, s); break;
      }
    } else {
      switch (bk) {
        case 0: e = launch_attn_bv<0, true>(aa, bv, al, grid, s); break;
        case 1: e = launch_attn_bv<1, true>(aa, bv, al, grid, s); break;
        case 2: e = launch_attn_bv<2, true>(aa, bv, al, grid, s); break;
        default: e = launch_attn_bv<3, true>(aa, bv, al, grid, s); break;
      }
    }
    if (e != hipSuccess) return TQ_ERR_HIP;
  }
  if (phase == 0 || phase == 3) {
    MergeArgs ma{part, tq_rotation_matrix(vq), static_cast<const PrepHeader*>(vq->prep), out, Hq, Hkv, G, p.ngroups, p.nsplit};
    hipLaunchKernelGGL(merge_kernel, dim3(p.units * kMaxHeads), dim3(kD), 0, s, ma);
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

extern "C" int tq_decode_step(const tq_quantizer* kq, const tq_quantizer* vq, const void* k_new,
                              const void* v_new, int x_dtype, int64_t x_row_stride, const float* query,
                              int B, int Hq, int Hkv, const int32_t* ctx_lens, int64_t max_ctx,
                              const tq_packed* k_cache, const tq_packed* v_cache, float scale, float* out,
                              void* workspace, size_t ws_bytes, void* stream) {
  const StepRows r{k_new, v_new, x_dtype, x_row_stride};
  return decode_call(0, kq, vq, query, B, Hq, Hkv, ctx_lens, max_ctx, k_cache, v_cache, scale, out,
                     workspace, ws_bytes, stream, &r);
}

extern "C" int tq_decode_step_phase(int phase, const tq_quantizer* kq, const tq_quantizer* vq,
                                    const void* k_new, const void* v_new, int x_dtype, int64_t x_row_stride,
                                    const float* query, int B, int Hq, int Hkv, const int32_t* ctx_lens,
                                    int64_t max_ctx, const tq_packed* k_cache, const tq_packed* v_cache,
                                    float scale, float* out, void* workspace, size_t ws_bytes, void* stream) {
  if (phase < 1 || phase > 3) return TQ_ERR_INVALID_ARG;
  const StepRows r{k_new, v_new, x_dtype, x_row_stride};
  return decode_call(phase, kq, vq, query, B, Hq, Hkv, ctx_lens, max_ctx, k_cache, v_cache, scale, out,
                     workspace, ws_bytes, stream, &r);
}

// ---------------------------------------------------------------------------
// Decode attention with a library-owned workspace, for callers that cannot
// allocate device memory. Its workspace is `scratch`, a fixed array in the
// code object: every GPU the library runs on holds its own copy until the
// process ends, and every call on that GPU shares it.
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = size_t(TQ_STATIC_SCRATCH_BYTES);
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's `scratch` (in host code the
// array's name is only a stand-in for it), looked up once per device.
int current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return TQ_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return TQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return TQ_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return TQ_OK;
}

}  // namespace

extern "C" int tq_attn_decode_noalloc(const tq_quantizer* kq, const tq_quantizer* vq, const float* query,
                                      int B, int Hq, int Hkv, const int32_t* ctx_lens, int64_t max_ctx,
                                      const tq_packed* k_cache, const tq_packed* v_cache, float scale,
                                      float* out, void* stream) {
  // Every argument check first (a stand-in workspace address, never used),
  // including the shape's workspace against the scratch's size.
  void* const stand_in = reinterpret_cast<void*>(uintptr_t(256));
  int st = decode_call(0, kq, vq, query, B, Hq, Hkv, ctx_lens, max_ctx, k_cache, v_cache, scale, out, stand_in,
                       kStaticScratchBytes, stream, nullptr, true);
  if (st != TQ_OK) return st;
  void* ws = nullptr;
  st = current_scratch(&ws);
  if (st != TQ_OK) return st;
  return decode_call(0, kq, vq, query, B, Hq, Hkv, ctx_lens, max_ctx, k_cache, v_cache, scale, out, ws,
                     kStaticScratchBytes, stream);
}

namespace {

constexpr int kMaxChunks = 64;   // vectors of up to 8192 coordinates

// Workspace of a search: the query operands and per-split lists, then (for
// vectors of more than one chunk) the running partial scores, float[units·8][n].
size_t search_ws_bytes(int nq, int64_t n, int k, int chunks, size_t* partial_off) {
  const Plan p = make_plan(1, nq, 1, n);
  const size_t lists = p.part_off + size_t(p.units) * p.nsplit * kMaxHeads * k * sizeof(uint64_t);
  const size_t poff = (lists + 255) / 256 * 256;
  if (partial_off != nullptr) *partial_off = poff;
  return chunks > 1 ? poff + size_t(p.units) * kMaxHeads * size_t(n) * sizeof(float) : lists;
}

bool search_sizes_ok(int nq, int64_t n, int k, int chunks) {
  return nq >= 1 && n >= 1 && n <= kMaxCtx && k >= 1 && k <= kSearchMaxK && k <= n && chunks >= 1 &&
         chunks <= kMaxChunks;
}

// One search over vectors of `chunks` 128-coordinate chunks, chunk c of vector
// v in slot c·n + v of db. Pass c takes the query operands of the queries'
// chunk c and scans chunk c's vectors; the scores of passes 0..chunks-2 go to
// the partial buffer, and the last pass adds them and keeps the candidates.
int search_call(const tq_quantizer* q, const float* query, int nq, int chunks, const tq_packed* db, int64_t n,
                int k, float* scores, int64_t* index, void* workspace, size_t ws_bytes, void* stream) {
  const int st = tq_check_quantizer(q);
  if (st != TQ_OK) return st;
  if (q->split != TQ_SPLIT_NONE) return TQ_ERR_UNSUPPORTED;
  if (query == nullptr || db == nullptr || scores == nullptr || index == nullptr || workspace == nullptr)
    return TQ_ERR_INVALID_ARG;
  if (nq < 1 || n < 1 || k < 1 || k > n || chunks < 1) return TQ_ERR_INVALID_ARG;
  if (k > kSearchMaxK || n > kMaxCtx || chunks > kMaxChunks) return TQ_ERR_UNSUPPORTED;
  const bool prod = q->variant == TQ_PROD;
  const int bk = prod ? q->bits - 1 : q->bits;
  if (db->norms == nullptr || (bk > 0 && db->codes == nullptr)) return TQ_ERR_INVALID_ARG;
  if (prod && (db->qjl == nullptr || db->gammas == nullptr)) return TQ_ERR_INVALID_ARG;
  if (!aligned(query, 16) || (bk > 0 && !aligned(db->codes, 16)) || !aligned(db->norms, 4) ||
      (prod && (!aligned(db->qjl, 16) || !aligned(db->gammas, 4))))
    return TQ_ERR_INVALID_ARG;
  const Plan p = make_plan(1, nq, 1, n);
  size_t poff = 0;
  const size_t need = search_ws_bytes(nq, n, k, chunks, &poff);
  if (ws_bytes < need || !aligned(workspace, 256)) return TQ_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const PrepHeader* kh = static_cast<const PrepHeader*>(q->prep);
  const bool al = (n % kBlockTok) == 0;
  const dim3 grid(p.nsplit, p.units);
  const size_t code_row = size_t(kD) * bk / 8;
  for (int c = 0; c < chunks; ++c) {
    // query operands of chunk c with log2(e)·scale = 1: the scores are plain
    // inner products
    PrepArgs pa{query + size_t(c) * kD, tq_rotation_matrix(q), tq_projection_matrix(q), kh, 0.69314718055994531f, nq, 1, nq,
                p.ngroups, p.units, ws, int64_t(chunks) * kD};
    hipLaunchKernelGGL(query_prep_kernel, dim3(p.units), dim3(kRowWaves * 64), 0, s, pa);
    if (hipGetLastError() != hipSuccess) return TQ_ERR_HIP;
    const size_t row0 = size_t(c) * size_t(n);
    SearchArgs sa;
    sa.kc = bk > 0 ? db->codes + row0 * code_row : nullptr;
    sa.kn = db->norms + row0;
    sa.kq = prod ? db->qjl + row0 * (kD / 8) : nullptr;
    sa.kg = prod ? db->gammas + row0 : nullptr;
    sa.n = n;
    sa.kcent = q->centroids;
    sa.kh = kh;
    sa.ws = ws;
    sa.part = reinterpret_cast<uint64_t*>(ws + p.part_off);
    sa.ngroups = p.ngroups;
    sa.nq = nq;
    sa.nsplit = p.nsplit;
    sa.split_len = p.split_len;
    sa.k = k;
    sa.partial = chunks > 1 ? reinterpret_cast<float*>(ws + poff) : nullptr;
    sa.pin = c > 0;
    sa.pout = c + 1 < chunks;
    hipError_t e;
    if (!prod) {
      switch (bk) {
        case 1: e = launch_search_t<1, false>(sa, al, grid, s); break;
        case 2: e = launch_search_t<2, false>(sa, al, grid, s); break;
        case 3: e = launch_search_t<3, false>(sa, al, grid, s); break;
        default: e = launch_search_t<4, false>(sa, al, grid, s); break;
      }
    } else {
      switch (bk) {
        case 0: e = launch_search_t<0, true>(sa, al, grid, s); break;
        case 1: e = launch_search_t<1, true>(sa, al, grid, s); break;
        case 2: e = launch_search_t<2, true>(sa, al, grid, s); break;
        default: e = launch_search_t<3, true>(sa, al, grid, s); break;
      }
    }
    if (e != hipSuccess) return TQ_ERR_HIP;
  }
  hipLaunchKernelGGL(search_merge_kernel, dim3(nq), dim3(kDecWaves * 64), 0, s,
                     reinterpret_cast<uint64_t*>(ws + p.part_off), p.nsplit, k, scores, index);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

}  // namespace

extern "C" size_t tq_search_workspace(int nq, int64_t n, int k) {
  return search_sizes_ok(nq, n, k, 1) ? search_ws_bytes(nq, n, k, 1, nullptr) : 0;
}

extern "C" int tq_search(const tq_quantizer* q, const float* query, int nq, const tq_packed* db, int64_t n, int k,
                         float* scores, int64_t* index, void* workspace, size_t ws_bytes, void* stream) {
  return search_call(q, query, nq, 1, db, n, k, scores, index, workspace, ws_bytes, stream);
}

extern "C" size_t tq_search_chunked_workspace(int nq, int64_t n, int k, int chunks) {
  return search_sizes_ok(nq, n, k, chunks) ? search_ws_bytes(nq, n, k, chunks, nullptr) : 0;
}

extern "C" int tq_search_chunked(const tq_quantizer* q, const float* query, int nq, int chunks, const tq_packed* db,
                                 int64_t n, int k, float* scores, int64_t* index, void* workspace, size_t ws_bytes,
                                 void* stream) {
  return search_call(q, query, nq, chunks, db, n, k, scores, index, workspace, ws_bytes, stream);
}

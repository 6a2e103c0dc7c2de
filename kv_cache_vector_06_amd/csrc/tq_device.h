// Device-side building blocks shared by the encode and decode kernels:
// matrix-core operand types, the 16x16x32 fp16 MFMA, lane helpers and the
// fixed operand-layout constants. gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;           // head dimension
constexpr int kWave = 64;
constexpr float kCentScale = 64.0f;   // centroids enter fp16 tables as c·64·σ

// A quantizer's prepared buffer (written by tq_prepare): a 256-byte header,
// then two sets of matrix-core A operands, each 2 parts (fp16 hi, lo) × 8 row
// tiles × 4 K-steps × 64 lanes × 16 bytes: rot_scale·Π, and (prod) S' = S·Πᵀ
// scaled by the power of two sp_scale. Fragment (part, t, s), lane (i, g), slot j
// holds row out_row(t, i) and column 32s + 8g + j (16Π) or 32g + 8s + j (S').
constexpr size_t kPrepHeaderBytes = 256;
struct PrepHeader {
  float sigma;       // centroid scale σ in [1, 2), see prepare_kernel
  float sigma_err;   // max relative fp16 error of c·64·σ over the centroids
  float sp_scale;    // the power of two S' is scaled by in its fragments
  float rot_scale;   // the rotation fragments hold rot_scale·Π: 16 (dense Π, fp16
                     // hi + lo), or √d for a randomized Hadamard Π = H·diag(s)/√d,
                     // whose fragments H·diag(s) are exact ±1 (lo parts zero)
  uint32_t omask[4]; // outlier-channel split: bit c set when raw channel c is an
                     // outlier channel (its column of Π lies in the outlier rows)
};
constexpr int kFragsPerSet = 2 * 8 * 4;               // (part, t, s)
constexpr size_t kSetBytes = size_t(kFragsPerSet) * 64 * 16;  // 64 KiB
// Then float[d][d]: an outlier-channel split quantizer's whole rotation, the
// block-structured matrix tq_prepare builds from Π_o, Π_r and the channel list
// (rows p mod 8 < 2 hold Π_o over the outlier channels, the other rows Π_r
// over the regular channels); unused otherwise.
// A split prod quantizer's sketch matrix follows in the same structure
// (rows: sketch positions, columns: channels).
constexpr size_t kPrepRotOff = kPrepHeaderBytes + 2 * kSetBytes;
constexpr size_t kPrepProjOff = kPrepRotOff + size_t(kD) * kD * sizeof(float);
constexpr size_t kPrepBytes = kPrepProjOff + size_t(kD) * kD * sizeof(float);
constexpr float kRotScale = 16.0f;                    // dense Π: |Π| <= 1 → |16Π| <= 16
constexpr float kResScale = 64.0f;                    // residual scale of the sketch operand

__host__ __device__ constexpr int frag_index(int part, int t, int s) { return (part * 8 + t) * 4 + s; }

// Output row held by A-row i of row tile t: lane group i/4 ends up holding
// rows 32*(i/4) + 4t + (i%4), so each lane group owns 32 consecutive outputs.
__device__ __forceinline__ int out_row(int t, int i) { return 32 * (i >> 2) + 4 * t + (i & 3); }

// D(16x16, fp32) += A(16x32, fp16) · B(32x16, fp16).
// Lane l holds row l%16 of A and column l%16 of B, both over the K-slice of
// lane group l/16; the result row 4*(l/16)+i, column l%16 sits in element i.
__device__ __forceinline__ f32x4 mfma(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

// A load through the scalar unit (uniform address, read-only data): its wait
// does not include the vector memory loads in flight.
template <typename T>
__device__ __forceinline__ T scalar_load(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

__device__ __forceinline__ uint16_t f2h_bits(float x) {  // round to nearest even
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}
__device__ __forceinline__ float h2f(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}
__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
  return static_cast<uint32_t>(f2h_bits(lo)) | (static_cast<uint32_t>(f2h_bits(hi)) << 16);
}

// fp16 split of a float: x ≈ hi + lo with both halves fp16 (≈22-bit mantissa).
__device__ __forceinline__ void split_h(float x, uint16_t& hi, uint16_t& lo) {
  hi = f2h_bits(x);
  lo = f2h_bits(x - h2f(hi));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }

// Reduce over the four lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float sum4g(float v) {
  v += shfl_xor_f(v, 16);
  v += shfl_xor_f(v, 32);
  return v;
}
__device__ __forceinline__ float max4g(float v) {
  v = fmaxf(v, shfl_xor_f(v, 16));
  v = fmaxf(v, shfl_xor_f(v, 32));
  return v;
}

// Scale of a row for its fp16 matrix-core operand. Each lane holds 32 of the
// row's 128 values (xv; the row spans lane groups l, l^16, l^32, l^48) and ss
// is the row's sum of squares. fp32 rows, and bf16 rows with ss outside
// [1, 2^31), are scaled by 2^-ex with max|x| = m·2^ex, m in [0.5, 1): the
// squares can then neither overflow nor vanish (xv and ss are replaced by the
// scaled values). A bf16 row with ss in [1, 2^31) is used as it is (ex = 0):
// every component is below 2^15.5, so its fp16 form is exact except where it
// is an fp16 subnormal (below 2^-14), off by at most 2^-25, under 2^-25 of
// the row's norm. Scaling by a power of two changes no code, norm or sketch
// bit: the products, thresholds and residuals scale with it exactly.
template <bool F32IN>
__device__ __forceinline__ int row_exponent(float (&xv)[32], float& ss) {
  int ex = 0;
  if (F32IN || !(ss >= 1.0f && ss < 0x1p31f)) {
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < 32; ++q) amax = fmaxf(amax, fabsf(xv[q]));
    amax = max4g(amax);
    if (amax > 0.f) frexpf(amax, &ex);
    ss = 0.f;
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      xv[q] = ldexpf(xv[q], -ex);    // a zero row stays ±0 (ex = 0)
      ss = fmaf(xv[q], xv[q], ss);
    }
    ss = sum4g(ss);
  }
  return ex;
}

// fp16 pair of two values of a bf16 row (unscaled or scaled by a power of
// two): the conversion is exact unless a value is an fp16 subnormal, so one
// packed round-toward-zero conversion serves (the same in every encoder).
__device__ __forceinline__ uint32_t bf16_row_pair(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// Sum of squares of a bf16 row (0 for fp32 rows: row_exponent computes it).
template <bool F32IN>
__device__ __forceinline__ float row_ss(const float (&xv)[32]) {
  float ss = 0.f;
  if constexpr (!F32IN) {
#pragma unroll
    for (int q = 0; q < 32; ++q) ss = fmaf(xv[q], xv[q], ss);
    ss = sum4g(ss);
  }
  return ss;
}

}  // namespace tq

// Measurement aid, not a step of the codec: one plain coalesced read of a
// device buffer, with the 16-byte non-temporal loads the decode kernels use
// for the packed cache. Its rate on a buffer far larger than the last-level
// cache is the part's practical read ceiling, against which the decode rate
// can be set beside the published 8 TB/s. The XOR of the buffer's 32-bit
// words is its only output, so the read cannot be elided and can be checked.
#include <hip/hip_runtime.h>

#include "tq.h"
#include "tq_device.h"

namespace tq {

// Two workgroups of four wavefronts per compute unit, four 16-byte loads in
// flight per lane (32 KiB per compute unit): on gfx950 this reads fastest of
// the shapes tried (≈7.1 TB/s over 4 GiB). Half the loads in flight reach only
// ≈4 TB/s, and more workgroups per compute unit are slower again.
constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;
constexpr int kProbeBlocksPerCU = 2;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ p, size_t n16,
                                                                    uint32_t* __restrict__ xor_out) {
  const size_t stride = size_t(gridDim.x) * kProbeThreads;
  size_t i = size_t(blockIdx.x) * kProbeThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  // Grid-stride: each round of the grid reads one contiguous stretch.
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int m = kWave / 2; m >= 1; m >>= 1) x ^= __shfl_xor(x, m, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) atomicXor(xor_out, x);
}

}  // namespace tq

using namespace tq;

extern "C" int tq_read_probe(const void* buf, size_t bytes, uint32_t* xor_out, void* stream) {
  if (!buf || !xor_out || (reinterpret_cast<uintptr_t>(buf) & 15) || (reinterpret_cast<uintptr_t>(xor_out) & 3) ||
      bytes == 0 || (bytes & 15))
    return TQ_ERR_INVALID_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess)
    return TQ_ERR_HIP;
  const size_t n16 = bytes / 16;
  const size_t per_round = size_t(kProbeThreads) * kProbeUnroll;
  size_t grid = size_t(cus) * kProbeBlocksPerCU;
  const size_t need = (n16 + per_round - 1) / per_round;   // no idle workgroups on small buffers
  if (grid > need) grid = need;
  hipLaunchKernelGGL(read_probe_kernel, dim3(unsigned(grid)), dim3(kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf), n16, xor_out);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

// Probes for benchmarks, so the attainable rates of the device can be measured beside
// the published peaks: waves that issue only 32x32x16 bf16 MFMAs (no memory traffic
// inside the timed loop), and a read-only stream over a device buffer.
#include "zaya.h"
#include "common.h"

namespace zaya {
namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;
constexpr int kProbeChains = 8;  // independent accumulators per wave: covers the MFMA latency
constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(int iters, float* __restrict__ sink) {
  const uint32_t gid = blockIdx.x * kProbeThreads + threadIdx.x;
  // varied nonzero operand bits (bf16 values of magnitude ~1 with mixed signs and mantissas)
  uint32_t h = gid * 0x9E3779B9u + 0x7F4A7C15u;
  uint4 a, b;
  uint32_t* pa = reinterpret_cast<uint32_t*>(&a);
  uint32_t* pb = reinterpret_cast<uint32_t*>(&b);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h ^= h << 13; h ^= h >> 17; h ^= h << 5;
    pa[i] = (h & 0x807F807Fu) | 0x3F003F00u;
    h ^= h << 13; h ^= h >> 17; h ^= h << 5;
    pb[i] = (h & 0x807F807Fu) | 0x3F003F00u;
  }
  const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a), bv = __builtin_bit_cast(bf16x8_t, b);
  f32x16 acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[c], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[gid] = s;
}

// Read-only stream: each thread loads 16-byte chunks in a grid-stride loop (the
// grid's loads of one pass are contiguous), non-temporal, folded into one word.
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint4* __restrict__ src, size_t n16,
                                                                   float* __restrict__ sink) {
  const size_t gid = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  u32x4 acc = u32x4{0u, 0u, 0u, 0u};
  size_t i = gid;
  for (; i + 3 * stride < n16; i += 4 * stride) {  // four loads in flight per thread
    const u32x4 v0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + i));
    const u32x4 v1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + i + stride));
    const u32x4 v2 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + i + 2 * stride));
    const u32x4 v3 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + i + 3 * stride));
    acc ^= v0 ^ v1 ^ v2 ^ v3;
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + i));
  sink[gid] = __uint_as_float(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
}

}  // namespace
}  // namespace zaya

extern "C" int zaya_probe_mfma_bf16(int n_wg, int iters, float* sink, void* stream, double* flops) {
  if (n_wg <= 0 || iters <= 0 || !sink) return ZAYA_EINVAL;
  hipLaunchKernelGGL(zaya::mfma_probe_kernel, dim3(n_wg), dim3(zaya::kProbeThreads), 0, (hipStream_t)stream, iters,
                     sink);
  if (hipGetLastError() != hipSuccess) return ZAYA_EHIP;
  // per wave and iteration: kProbeChains MFMAs of 32 x 32 x 16 multiply-adds
  if (flops) *flops = (double)n_wg * (zaya::kProbeThreads / 64) * iters * zaya::kProbeChains * (2.0 * 32 * 32 * 16);
  return 0;
}

extern "C" int zaya_probe_hbm_read(const void* src, size_t bytes, int n_wg, float* sink, void* stream) {
  if (!src || !sink || n_wg <= 0 || bytes < 16 || (bytes & 15) || ((uintptr_t)src & 15)) return ZAYA_EINVAL;
  hipLaunchKernelGGL(zaya::read_probe_kernel, dim3(n_wg), dim3(zaya::kProbeThreads), 0, (hipStream_t)stream,
                     reinterpret_cast<const uint4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : ZAYA_EHIP;
}

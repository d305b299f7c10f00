// Matrix-core throughput probe: the sustained rate of v_mfma_f32_32x32x16_bf16 on
// this GPU for a given kind of operand data. It is a measurement helper beside the
// attention kernels, so that their achieved rate can be read against what the matrix
// cores sustain at the clock the chip actually runs, not only against the
// datasheet peak (256 CUs x 2.4 GHz x 4096 flop/clk).
//
// Each wave keeps 16 A and 8 B operands in registers and runs `iters` rounds of 16
// products into two accumulators; nothing else is in the loop. The operand values
// matter: the clock the chip sustains under matrix load depends on how many
// multiplier bits toggle, so the probe can fill them with zeros or with bf16
// values drawn from an approximately standard normal distribution (the value
// distribution of the attention workloads' Q, K and V).
#include "common.h"
#include "kernels.h"

namespace fa {
namespace {

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Approximately N(0,1): the sum of four uniforms on [0,1) has mean 2 and variance
// 1/3, so (sum - 2) * sqrt(3) has unit variance.
__device__ __forceinline__ float normalish(uint32_t key) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += (float)(mix32(key * 4u + (uint32_t)i) >> 8) * (1.f / 16777216.f);
  return (s - 2.f) * 1.7320508f;
}

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);  // round to nearest even
}

template <int KIND>
__global__ __launch_bounds__(256) void mfma_probe_kernel(float* out, int iters, uint32_t seed) {
  bf16x8_t a[16], b[8];
  const uint32_t base = seed ^ (blockIdx.x * 256u + threadIdx.x) * 0x9e3779b9u;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    u32x4_t w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t k = base + (uint32_t)(16 * j + 2 * e) * 0x85ebca6bu;
      w[e] = KIND == 0 ? 0u
                       : (uint32_t)to_bf16_bits(normalish(k)) |
                             ((uint32_t)to_bf16_bits(normalish(k + 0x27d4eb2fu)) << 16);
    }
    a[j] = __builtin_bit_cast(bf16x8_t, w);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    u32x4_t w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t k = base + (uint32_t)(1000 + 16 * j + 2 * e) * 0xc2b2ae35u;
      w[e] = KIND == 0 ? 0u
                       : (uint32_t)to_bf16_bits(normalish(k)) |
                             ((uint32_t)to_bf16_bits(normalish(k + 0x165667b1u)) << 16);
    }
    b[j] = __builtin_bit_cast(bf16x8_t, w);
  }
  f32x16_t acc0 = zero16(), acc1 = zero16();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc0 = mfma32x32x16(a[2 * j], b[j], acc0);
      acc1 = mfma32x32x16(a[2 * j + 1], b[j], acc1);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += acc0[r] + acc1[r];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_probe(float* out, int blocks, int iters, int kind, hipStream_t st) {
  if (kind == 0)
    hipLaunchKernelGGL(mfma_probe_kernel<0>, dim3(blocks), dim3(256), 0, st, out, iters, 12345u);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<1>, dim3(blocks), dim3(256), 0, st, out, iters, 12345u);
  return hipGetLastError();
}

}  // namespace fa

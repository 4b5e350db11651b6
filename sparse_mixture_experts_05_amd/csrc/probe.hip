// Measurement probes (not part of the layer): the rate the matrix cores reach
// with no memory traffic at all, as context for the grouped GEMM's fraction of
// the datasheet peak. Built into libmoe_probe.so; declared in
// include/moe_probe.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_probe.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kChains = 8;  // independent accumulators per wave

// Every wave runs `iters` rounds of kChains independent
// v_mfma_f32_32x32x16_bf16 on register operands: 32*32*16*2 flops each, no
// loads, no LDS. Two workgroups of 4 waves per CU (2 waves per SIMD) keep each
// matrix core fed while a wave's dependent chain waits. The operands are small
// bf16 values derived from the lane id, so the sums stay finite; each thread
// writes the sum of its accumulators to sink, which keeps the work live.
__global__ __launch_bounds__(256, 2) void mfma_loop_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.0009765625f * (float)((lane + i) & 7));
    b[i] = (__bf16)(0.0009765625f * (float)((lane * 3 + i) & 7));
  }
  f32x16_t acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[c][v];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

double moe_probe_mfma_bf16_flops(int blocks, int iters) {
  return (double)blocks * 4.0 * (double)iters * kChains * (32.0 * 32.0 * 16.0 * 2.0);
}

int moe_probe_mfma_bf16(int blocks, int iters, float* sink, void* stream) {
  if (blocks < 1 || blocks > 65536 || iters < 1 || sink == nullptr) return -1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"

// Shared device helpers for the MoE layer kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
// 16-byte payload in registers (a native vector: arrays of it stay in VGPRs,
// unlike HIP's struct-wrapped uint4).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (NaN -> quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 -> packed pair of bf16 (low half = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return f32_to_bf16(a) | (f32_to_bf16(b) << 16);
}

// The same pair conversion in one instruction (v_cvt_pk_bf16_f32, round to
// nearest even; NaN stays a quiet NaN of its own sign and payload bits).
typedef __bf16 bf16x2_hw_t __attribute__((ext_vector_type(2)));
typedef float f32x2_hw_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  const f32x2_hw_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_hw_t));
}

// GeLU, erf form: 0.5 * a * (1 + erf(a / sqrt(2))). erff is the device library's.
__device__ __forceinline__ float gelu_erf(float a) {
  return 0.5f * a * (1.0f + erff(a * 0.70710678118654752f));
}

// GeLU (erf form) for bf16 outputs: 0.5 * a * (1 + erf(a / sqrt(2))) is
// a * Phi(a), Phi the standard normal distribution function. With u = |a| and
// q = Phi(-u), Phi(a) = 1 - q for a >= 0 and q for a < 0, so
// GeLU(a) = max(a, 0) - u * q on both sides. q = 2^p(u), p a degree-6
// polynomial fitted to log2 Phi(-u) on [0, 6] (near-minimax,
// |p - log2 Phi(-u)| <= 6.5e-5, so q is within 4.5e-5 of Phi(-u) relative;
// csrc/gelu_fit.py derives the coefficients). u is clamped at 6, where
// Phi(-6) = 1e-9: past |a| = 6 the result is max(a, 0) - 6 * Phi(-6), within
// 6e-9 of the exact value. One exp2 and no division: the relative error of the
// result stays within about 5e-5, far below the bf16 step (2^-8) it is rounded
// to. Per element the VALU runs one med3 (the clamp, |a| a source modifier),
// six FMAs, the exp2, a compare and select (max(a, 0) that keeps a NaN) and
// one FMA. NaN stays NaN, +inf stays +inf.
__device__ __forceinline__ float gelu_bf16(float a) {
  const float u = __builtin_amdgcn_fmed3f(fabsf(a), 0.0f, 6.0f);
  float p = fmaf(2.29900634e-05f, u, -0.000611100055f);
  p = fmaf(p, u, 0.00719556585f);
  p = fmaf(p, u, -0.051185336f);
  p = fmaf(p, u, -0.461271912f);
  p = fmaf(p, u, -1.15017426f);
  p = fmaf(p, u, -1.00006473f);
  const float q = __builtin_amdgcn_exp2f(p);  // p in [-30, -1]: no range reduction needed
  const float r = !(a <= 0.0f) ? a : 0.0f;    // a NaN passes through
  return fmaf(-u, q, r);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }

// Wait until at most N global loads of this wave are outstanding (they
// complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for LDS hand-off only. __syncthreads() carries a release
// fence that waits for every outstanding global load (vmcnt 0), which would
// drain the next stage's prefetch; the staged loads are waited for explicitly.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// global_load_lds_dwordx4: lane i copies 16 bytes from its address g into
// LDS at M0 + 16*i (M0 = the wave-uniform LDS address). Issued through asm so
// the compiler's wait insertion does not treat every later LDS read as
// aliasing the in-flight copy (which would drain the prefetch); completion is
// tracked with explicit vmcnt waits (loads complete in issue order).
__device__ __forceinline__ void lds_dma16(const void* g, void* lds_uniform) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t*)(lds_uniform))));
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(g), "s"(m0)
      : "memory");
}

// Value of the partner lane of butterfly level L: xor 1, xor 2, the mirror
// lane within 8, within 16 (DPP), xor 16 (ds_swizzle), xor 32 (bpermute).
// Each level pairs two groups that the earlier levels already merged.
template <int L>
__device__ __forceinline__ uint32_t partner(uint32_t v) {
  if constexpr (L == 0) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
  if constexpr (L == 1) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
  if constexpr (L == 2) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);
  if constexpr (L == 3) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false);
  if constexpr (L == 4) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
  if constexpr (L == 5)
    return (uint32_t)__builtin_amdgcn_ds_bpermute((int)(((threadIdx.x & 63) ^ 32) * 4), (int)v);
  return v;
}
template <int L>
__device__ __forceinline__ uint64_t partner64(uint64_t v) {
  return ((uint64_t)partner<L>((uint32_t)(v >> 32)) << 32) | partner<L>((uint32_t)v);
}

}  // namespace moe

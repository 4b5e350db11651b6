// Step 4 - weighted combine back to the original token order.
//
// Method: "hncyxsy.com Kimi K3 fine-grained MoE" article, combine phase (the
// expert outputs return to the token's owner and are summed with the routing
// weights) and "lpqz.cn MoE engineering blog" section 3.1 (results are
// scattered back to the original positions); the always-on shared expert's
// row is added with weight 1.
//
// One wavefront per token (per column segment of the token's row when there
// are few tokens). The token's k buffer rows are found through inv
// (a gather, so every output row is written exactly once: no atomics, and a
// fixed summation order j = 0..k-1, then the shared row). An assignment that
// a capacity dropped (inv < 0) is skipped; the other weights are kept as they
// are (no renormalisation). 16-byte loads and stores; fp32 accumulation in
// registers.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void fma_bf16x8(float (&acc)[8], uint4 v, float w) {
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc[2 * q] = fmaf(w, bf16_to_f32(u[q] & 0xffffu), acc[2 * q]);
    acc[2 * q + 1] = fmaf(w, bf16_to_f32(u[q] >> 16), acc[2 * q + 1]);
  }
}

__device__ __forceinline__ void add_bf16x8(float (&acc)[8], uint4 v) {
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc[2 * q] += bf16_to_f32(u[q] & 0xffffu);
    acc[2 * q + 1] += bf16_to_f32(u[q] >> 16);
  }
}

// Loads and stores of rows touched once. NT: non-temporal (the rows stream
// past the caches instead of evicting lines that are still of use), for
// buffers well beyond the 256 MB last-level cache.
template <bool NT>
__device__ __forceinline__ uint4 ld_row(const uint4* p) {
  if constexpr (NT)
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
  else
    return *p;
}
template <bool NT>
__device__ __forceinline__ void st_row(uint4* p, uint4 v) {
  if constexpr (NT)
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v), reinterpret_cast<u32x4_t*>(p));
  else
    *p = v;
}

// bf16: each 16-byte vector holds 8 values. KM >= k (a power of two); U = 8/KM
// column steps are loaded before any is summed, so about 8 16-byte loads per
// lane are in flight whatever k is.
template <int KM, bool NT>
__global__ __launch_bounds__(kThreads) void combine_bf16_kernel(
    const uint4* __restrict__ ys, const int32_t* __restrict__ inv, const float* __restrict__ w,
    const uint4* __restrict__ ysh, int T, int vpr, int k, int seg, uint4* __restrict__ out) {
  constexpr int U = 8 / KM;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kThreads / kWave) + (threadIdx.x >> 6);
  if (t >= T) return;
  // this wave's columns: segment blockIdx.y of the row (one segment when T is large)
  const int cbeg = blockIdx.y * seg, cend = min(vpr, cbeg + seg);
  int row[KM];
  float wt[KM];
  bool keep[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const int r = j < k ? inv[(size_t)t * k + j] : -1;
    keep[j] = r >= 0;  // a dropped assignment (inv < 0) adds nothing
    row[j] = min(max(r, 0), T * k - 1);
    wt[j] = j < k ? w[(size_t)t * k + j] : 0.0f;
  }
  // The wave works on one token, so which slots are kept is the same on
  // every lane: a scalar test picks the load form.
  int kmask = 0;
#pragma unroll
  for (int j = 0; j < KM; ++j) kmask |= keep[j] ? 1 << j : 0;
  const bool all_kept = __builtin_amdgcn_readfirstlane(kmask) == (1 << KM) - 1;
  for (int c0 = cbeg + lane; c0 < cend; c0 += U * kWave) {
    uint4 v[U][KM], sh[U];
    if (all_kept) {
      // every load unconditional, from a column clamped into the segment, so
      // all U * KM loads are in flight before the first wait
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = min(c0 + u * kWave, cend - 1);
#pragma unroll
        for (int j = 0; j < KM; ++j) v[u][j] = ld_row<NT>(&ys[(size_t)row[j] * vpr + c]);
        if (ysh != nullptr) sh[u] = ld_row<NT>(&ysh[(size_t)t * vpr + c]);
      }
    } else {
      // dropped or padding slots (k below KM): load only the kept rows
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * kWave;
        if (c < cend) {
#pragma unroll
          for (int j = 0; j < KM; ++j)
            if (keep[j]) v[u][j] = ld_row<NT>(&ys[(size_t)row[j] * vpr + c]);
          if (ysh != nullptr) sh[u] = ld_row<NT>(&ysh[(size_t)t * vpr + c]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave;
      if (c < cend) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KM; ++j)
          if (keep[j]) fma_bf16x8(acc, v[u][j], wt[j]);
        if (ysh != nullptr) add_bf16x8(acc, sh[u]);
        uint4 o;
        // one v_cvt_pk_bf16_f32 per pair (round to nearest even, the same
        // bits as the software rounding except NaN payloads): with k = 8 the
        // software form's VALU work cost 3.5 us of 65 on the fine-grained layer
        o.x = cvt_bf16x2(acc[0], acc[1]);
        o.y = cvt_bf16x2(acc[2], acc[3]);
        o.z = cvt_bf16x2(acc[4], acc[5]);
        o.w = cvt_bf16x2(acc[6], acc[7]);
        st_row<NT>(&out[(size_t)t * vpr + c], o);
      }
    }
  }
}

// fp32: each 16-byte vector holds 4 values.
__global__ __launch_bounds__(kThreads) void combine_f32_kernel(
    const float4* __restrict__ ys, const int32_t* __restrict__ inv, const float* __restrict__ w,
    const float4* __restrict__ ysh, int T, int vpr, int k, int seg, float4* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kThreads / kWave) + (threadIdx.x >> 6);
  if (t >= T) return;
  const int cbeg = blockIdx.y * seg, cend = min(vpr, cbeg + seg);
  int row[8];
  float wt[8];
  bool keep[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = j < k ? inv[(size_t)t * k + j] : -1;
    keep[j] = r >= 0;  // a dropped assignment (inv < 0) adds nothing
    row[j] = min(max(r, 0), T * k - 1);
    wt[j] = j < k ? w[(size_t)t * k + j] : 0.0f;
  }
  for (int c = cbeg + lane; c < cend; c += kWave) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k && keep[j]) {
        const float4 v = ys[(size_t)row[j] * vpr + c];
        acc.x = fmaf(wt[j], v.x, acc.x);
        acc.y = fmaf(wt[j], v.y, acc.y);
        acc.z = fmaf(wt[j], v.z, acc.z);
        acc.w = fmaf(wt[j], v.w, acc.w);
      }
    }
    if (ysh != nullptr) {
      const float4 v = ysh[(size_t)t * vpr + c];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    out[(size_t)t * vpr + c] = acc;
  }
}

}  // namespace

hipError_t launch_combine(const void* ys, const int32_t* inv, const float* topk_w,
                          const void* ysh, int T, int H, int k, bool bf16, void* out,
                          hipStream_t s) {
  // Few tokens: split each row into column segments (grid.y) so that about
  // 1024 wavefronts stream the rows, each segment one pass of the wave.
  const int grid = (T + 3) / 4;
  const int vpr = H / (bf16 ? 8 : 4);
  const int km = k <= 1 ? 1 : k <= 2 ? 2 : k <= 4 ? 4 : 8;
  const int step = bf16 ? (8 / km) * kWave : kWave;  // vectors one pass of a wave covers
  int nseg = std::max(1, std::min((vpr + step - 1) / step, (1024 + T - 1) / T));
  const int seg = ((vpr + nseg - 1) / nseg + step - 1) / step * step;
  nseg = (vpr + seg - 1) / seg;
  if (bf16) {
    // expert rows beyond ~3/4 of the last-level cache: stream them (measured:
    // 1.07 GB of rows 254 -> 227 us, 268 MB 73 -> 70 us, 67 MB 18.2 -> 19.0 us)
    const bool nt = (size_t)T * k * H * 2 > (size_t(192) << 20);
    auto kern = km == 1   ? (nt ? combine_bf16_kernel<1, true> : combine_bf16_kernel<1, false>)
                : km == 2 ? (nt ? combine_bf16_kernel<2, true> : combine_bf16_kernel<2, false>)
                : km == 4 ? (nt ? combine_bf16_kernel<4, true> : combine_bf16_kernel<4, false>)
                          : (nt ? combine_bf16_kernel<8, true> : combine_bf16_kernel<8, false>);
    hipLaunchKernelGGL(kern, dim3(grid, nseg), dim3(kThreads), 0, s,
                       static_cast<const uint4*>(ys), inv, topk_w,
                       static_cast<const uint4*>(ysh), T, vpr, k, seg, static_cast<uint4*>(out));
  } else {
    hipLaunchKernelGGL(combine_f32_kernel, dim3(grid, nseg), dim3(kThreads), 0, s,
                       static_cast<const float4*>(ys), inv, topk_w,
                       static_cast<const float4*>(ysh), T, vpr, k, seg,
                       static_cast<float4*>(out));
  }
  return hipGetLastError();
}

}  // namespace moe

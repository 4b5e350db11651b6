// Step 1 - router gating: scores, softmax over experts, top-k, renormalisation.
//
// Method: "hncyxsy.com Kimi K3 fine-grained MoE" article, router listing
// (gate Linear without bias, softmax over all experts, top-k, divide the k
// weights by their sum) and "Kimi K3 专家路由不均衡诊断" section 4.2 (the
// per-expert bias B is added inside the softmax).
//
// The k renormalised weights are exp(s_j - m) / sum_j' exp(s_j' - m) with
// m = max_e s_e: the full-E softmax denominator cancels, so only the k chosen
// scores are exponentiated. Selection runs on the scores s (exp is monotone).
//
// Layout of the work: one workgroup of 256 threads owns BT tokens.
//   phase 1: scores [BT x E] into LDS. bf16: MFMA 16x16x32 tiles (tokens x
//            experts, K = H), fp32 accumulation, operands straight from
//            global memory (x rows are shared by the 4 waves through L1,
//            Wg comes from L2). fp32: plain dot products.
//   phase 2: one wavefront per token; every lane holds up to 4 scores
//            (E <= 256); k rounds of a wave-wide arg-max done in registers
//            with DPP (quad_perm, row mirrors) and ds_swizzle, lanes 0/32
//            merged with readlane. Ties go to the lower expert id.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxE = 256;
constexpr int kLogitStride = kMaxE + 4;  // LDS row stride (floats) of the score tile

__device__ __forceinline__ void take_better(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}

template <int CTRL>
__device__ __forceinline__ void dpp_step(float& v, int& i) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(0, i, CTRL, 0xF, 0xF, false);
  take_better(v, i, ov, oi);
}

// All 64 lanes end with the wave's best (v, i).
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  dpp_step<0xB1>(v, i);   // quad_perm [1,0,3,2]: lane ^ 1
  dpp_step<0x4E>(v, i);   // quad_perm [2,3,0,1]: lane ^ 2
  dpp_step<0x141>(v, i);  // row_half_mirror: pairs the two quads of each 8
  dpp_step<0x140>(v, i);  // row_mirror: pairs the two 8-lane halves of each row
  {                       // ds_swizzle bit-mask mode, xor 16: pairs the rows of each 32
    const float ov = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
    const int oi = __builtin_amdgcn_ds_swizzle(i, 0x401F);
    take_better(v, i, ov, oi);
  }
  const float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const int i0 = __builtin_amdgcn_readlane(i, 0);
  const float v1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const int i1 = __builtin_amdgcn_readlane(i, 32);
  v = v0;
  i = i0;
  take_better(v, i, v1, i1);
}

// Sum over the 64 lanes with the same exchange pattern as wave_argmax. Each
// step adds a lane's value and its partner's, and fp addition is commutative,
// so every lane ends with the same bits.
__device__ __forceinline__ float wave_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
}

// Best live slot of this lane. Slots that are out of range or already taken
// are dead and never win (a NaN score is read as -inf, so every live slot
// beats every dead one and the k ids are always distinct and < E).
__device__ __forceinline__ void lane_best(const float (&v)[4], unsigned alive, int lane, float& bv,
                                          int& bi) {
  bv = -INFINITY;
  bi = 0x7fffffff;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (alive & (1u << q)) {
      const int i = lane + 64 * q;
      if (v[q] > bv || bi == 0x7fffffff) {
        bv = v[q];
        bi = i;
      }
    }
}

// Phase 2: scores of BT tokens are in LDS (row-major, kLogitStride).
// When pp is not null, the full softmax p[t, e] = exp(s_e - m) / sum_e' exp(s_e' - m)
// of every token is also summed over the workgroup's tokens (per wave in
// token order, then the 4 waves in order) and pp[e] receives the sum. The
// score tile is reused for that reduction, so sc is clobbered.
__device__ __forceinline__ void topk_phase(float* sc, int BT, int t0, int T, int E, int k,
                                           const float* __restrict__ bias,
                                           int32_t* __restrict__ topk_idx,
                                           float* __restrict__ topk_w, float* __restrict__ pp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float b[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    b[q] = (bias != nullptr && e < E) ? bias[e] : 0.0f;
  }
  float pacc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int t = wave; t < BT; t += kThreads / kWave) {
    const int tok = t0 + t;
    if (tok >= T) break;
    float v[4];
    unsigned alive = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      const float s = e < E ? sc[t * kLogitStride + e] + b[q] : -INFINITY;
      v[q] = s == s ? s : -INFINITY;
      if (e < E) alive |= 1u << q;
    }
    float bv;
    int bi;
    lane_best(v, alive, lane, bv, bi);
    float sv[8];
    int si[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        float wv = bv;
        int wi = bi;
        wave_argmax(wv, wi);
        sv[j] = wv;
        si[j] = wi;
        if ((wi & 63) == lane) {
          alive &= ~(1u << (wi >> 6));
          lane_best(v, alive, lane, bv, bi);
        }
      }
    }
    const float m = sv[0];
    if (pp != nullptr) {
      // dead slots hold -inf and give 0; a token whose scores are all -inf or
      // NaN has no distribution and adds nothing
      float z[4], zs = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        z[q] = m > -INFINITY ? expf(v[q] - m) : 0.0f;
        zs += z[q];
      }
      const float Z = wave_sum(zs);
      if (Z > 0.0f) {
#pragma unroll
        for (int q = 0; q < 4; ++q) pacc[q] += z[q] / Z;
      }
    }
    float ex[8];
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        ex[j] = expf(sv[j] - m);
        sum += ex[j];
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k && lane == j) {
        topk_idx[(size_t)tok * k + j] = si[j];
        topk_w[(size_t)tok * k + j] = ex[j] / sum;
      }
    }
  }
  if (pp != nullptr) {
    __syncthreads();  // every wave is done with the score tile
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      if (e < E) sc[wave * kMaxE + e] = pacc[q];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kThreads)
      pp[e] = ((sc[e] + sc[kMaxE + e]) + sc[2 * kMaxE + e]) + sc[3 * kMaxE + e];
  }
}

// P[e] = (sum over workgroups b, ascending, of part[b][e]) / T, in double.
__global__ __launch_bounds__(kThreads) void prob_mean_kernel(const float* __restrict__ part,
                                                             int nb, int T, int E,
                                                             float* __restrict__ prob_mean) {
  for (int e = threadIdx.x; e < E; e += kThreads) {
    double s = 0.0;
    for (int b = 0; b < nb; ++b) s += (double)part[(size_t)b * E + e];
    prob_mean[e] = (float)(s / (double)T);
  }
}

// K loop of the score tiles: a ring of D register buffers keeps the operand
// loads of the next D-1 k-steps in flight while one step runs on the matrix
// cores (the loop is unrolled by D so every ring index is static).
template <int MC, int NCW, int D>
__device__ __forceinline__ void mfma_ring(const uint16_t* const (&arow)[MC],
                                          const uint16_t* const (&brow)[NCW], int s0, int nsteps,
                                          int stride, f32x4_t (&acc)[MC][NCW]) {
  u32x4_t ra[D][MC], rb[D][NCW];
#pragma unroll
  for (int u = 0; u < D; ++u) {
    const int s = s0 + u * stride;
    if (s < nsteps) {
#pragma unroll
      for (int r = 0; r < MC; ++r) ra[u][r] = ld16(arow[r] + s * 32);
#pragma unroll
      for (int c = 0; c < NCW; ++c) rb[u][c] = ld16(brow[c] + s * 32);
    }
  }
  for (int base = s0; base < nsteps; base += D * stride) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int s = base + u * stride;
      if (s < nsteps) {
#pragma unroll
        for (int r = 0; r < MC; ++r)
#pragma unroll
          for (int c = 0; c < NCW; ++c)
            acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ra[u][r]),
                                                                as_bf16x8(rb[u][c]), acc[r][c], 0, 0, 0);
        const int sn = s + D * stride;
        if (sn < nsteps) {
#pragma unroll
          for (int r = 0; r < MC; ++r) ra[u][r] = ld16(arow[r] + sn * 32);
#pragma unroll
          for (int c = 0; c < NCW; ++c) rb[u][c] = ld16(brow[c] + sn * 32);
        }
      }
    }
  }
}

// bf16 scores with MFMA. MC: 16-token row chunks per workgroup; NCW: 16-expert
// column chunks per wave; KSPLIT: 1 = each wave owns NCW column chunks over
// all of H, 4 = the 4 waves split the K steps (interleaved) and the partial
// tiles are summed in a fixed order.
template <int MC, int NCW, int KSPLIT>
__global__ __launch_bounds__(kThreads) void route_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg,
    const float* __restrict__ bias, int T, int H, int E, int k, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ ppart) {
  constexpr int BT = MC * 16;
  static_assert(BT * kLogitStride >= 4 * kMaxE, "score tile too small for the probability sums");
  __shared__ float sc[BT * kLogitStride];
  __shared__ float part[KSPLIT == 4 ? 4 * BT * 48 : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * BT;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const int c0 = KSPLIT == 4 ? 0 : wave * NCW * 16;  // first expert column of this wave

  const uint16_t* arow[MC];
#pragma unroll
  for (int r = 0; r < MC; ++r) arow[r] = x + (size_t)min(t0 + r * 16 + r16, T - 1) * H + kq;
  const uint16_t* brow[NCW];
#pragma unroll
  for (int c = 0; c < NCW; ++c) brow[c] = wg + (size_t)min(c0 + c * 16 + r16, E - 1) * H + kq;

  f32x4_t acc[MC][NCW];
#pragma unroll
  for (int r = 0; r < MC; ++r)
#pragma unroll
    for (int c = 0; c < NCW; ++c) acc[r][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const bool active = KSPLIT == 4 || c0 < E;
  if (active) {
    const int nsteps = H / 32;
    const int s0 = KSPLIT == 4 ? wave : 0;
    mfma_ring<MC, NCW, (MC + NCW <= 4 ? 8 : 4)>(arow, brow, s0, nsteps, KSPLIT, acc);
  }
  // D layout of 16x16: lane holds column lane%16, rows (lane/16)*4 + v.
  if (KSPLIT == 1) {
    if (active) {
#pragma unroll
      for (int r = 0; r < MC; ++r)
#pragma unroll
        for (int c = 0; c < NCW; ++c) {
          const int col = c0 + c * 16 + r16;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = r * 16 + (lane >> 4) * 4 + v;
            if (col < E) sc[row * kLogitStride + col] = acc[r][c][v];
          }
        }
    }
    __syncthreads();
  } else {
#pragma unroll
    for (int r = 0; r < MC; ++r)
#pragma unroll
      for (int c = 0; c < NCW; ++c)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = r * 16 + (lane >> 4) * 4 + v;
          part[(wave * BT + row) * 48 + c * 16 + r16] = acc[r][c][v];
        }
    __syncthreads();
    for (int p = threadIdx.x; p < BT * E; p += kThreads) {
      const int row = p / E, col = p % E;
      float s = part[(0 * BT + row) * 48 + col];
      s += part[(1 * BT + row) * 48 + col];
      s += part[(2 * BT + row) * 48 + col];
      s += part[(3 * BT + row) * 48 + col];
      sc[row * kLogitStride + col] = s;
    }
    __syncthreads();
  }
  topk_phase(sc, BT, t0, T, E, k, bias, topk_idx, topk_w,
             ppart != nullptr ? ppart + (size_t)blockIdx.x * E : nullptr);
}

// fp32 scores with plain dot products (small fp32 layers).
__global__ __launch_bounds__(kThreads) void route_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wg, const float* __restrict__ bias,
    int T, int H, int E, int k, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ ppart) {
  constexpr int BT = 16;
  __shared__ float sc[BT * kLogitStride];
  const int t0 = blockIdx.x * BT;
  for (int p = threadIdx.x; p < BT * E; p += kThreads) {
    const int t = p / E, e = p % E;
    const float4* xr = reinterpret_cast<const float4*>(x + (size_t)min(t0 + t, T - 1) * H);
    const float4* wr = reinterpret_cast<const float4*>(wg + (size_t)e * H);
    float s = 0.0f;
    for (int h = 0; h < H / 4; ++h) {
      const float4 a = xr[h], b = wr[h];
      s = fmaf(a.x, b.x, s);
      s = fmaf(a.y, b.y, s);
      s = fmaf(a.z, b.z, s);
      s = fmaf(a.w, b.w, s);
    }
    sc[t * kLogitStride + e] = s;
  }
  __syncthreads();
  topk_phase(sc, BT, t0, T, E, k, bias, topk_idx, topk_w,
             ppart != nullptr ? ppart + (size_t)blockIdx.x * E : nullptr);
}


// Few tokens (decode-like): one workgroup per 16 tokens cannot stream Wg fast
// enough, so the scores are computed in two launches. Phase 1: one wavefront
// per (16 tokens, 16 experts, K slice) writes a partial score tile into the
// workspace ws[ks][t][e]. Phase 2: one wavefront per token sums its K slices
// in a fixed order (ks ascending), adds the bias and runs the top-k.
__global__ __launch_bounds__(64) void route_partial_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ wg,
                                                           int T, int H, int E, int ksteps,
                                                           float* __restrict__ ws) {
  const int lane = threadIdx.x;
  const int t0 = blockIdx.x * 16, e0 = blockIdx.y * 16, ks = blockIdx.z;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const int s0 = ks * ksteps;
  const uint16_t* const arow[1] = {x + (size_t)min(t0 + r16, T - 1) * H + kq + s0 * 32};
  const uint16_t* const brow[1] = {wg + (size_t)min(e0 + r16, E - 1) * H + kq + s0 * 32};
  f32x4_t acc[1][1] = {{f32x4_t{0.f, 0.f, 0.f, 0.f}}};
  mfma_ring<1, 1, 8>(arow, brow, 0, ksteps, 1, acc);
  const int e = e0 + r16;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int t = t0 + (lane >> 4) * 4 + v;
    if (t < T && e < E) ws[((size_t)ks * T + t) * E + e] = acc[0][0][v];
  }
}

__global__ __launch_bounds__(kThreads) void route_select_kernel(const float* __restrict__ ws,
                                                                const float* __restrict__ bias,
                                                                int T, int E, int k, int nks,
                                                                int32_t* __restrict__ topk_idx,
                                                                float* __restrict__ topk_w,
                                                                float* __restrict__ ppart) {
  constexpr int BT = kThreads / kWave;  // 4 tokens per workgroup
  __shared__ float sc[BT * kLogitStride];
  const int t0 = blockIdx.x * BT;
  for (int p = threadIdx.x; p < BT * E; p += kThreads) {
    const int t = p / E, e = p % E;
    if (t0 + t < T) {
      float s = 0.0f;
      for (int q = 0; q < nks; ++q) s += ws[((size_t)q * T + t0 + t) * E + e];
      sc[t * kLogitStride + e] = s;
    }
  }
  __syncthreads();
  topk_phase(sc, BT, t0, T, E, k, bias, topk_idx, topk_w,
             ppart != nullptr ? ppart + (size_t)blockIdx.x * E : nullptr);
}

// K slices for the two-phase path: enough wavefronts to spread the Wg read
// over the chip (about 1024), a power of two that divides H/32.
int route_kslices(int T, int H, int E) {
  const int tiles = ((T + 15) / 16) * ((E + 15) / 16);
  int ks = 1;
  while (ks * 2 * tiles <= 1024 && (H / 32) % (ks * 2) == 0 && ks * 2 <= 64) ks *= 2;
  return ks;
}

bool route_two_phase(int T, bool bf16) { return bf16 && T < 2048; }

template <int MC, int NCW, int KSPLIT>
hipError_t launch_bf16(const void* x, const void* wg, const float* bias, int T, int H, int E,
                       int k, int32_t* idx, float* w, float* pp, hipStream_t s) {
  const int grid = (T + MC * 16 - 1) / (MC * 16);
  hipLaunchKernelGGL((route_bf16_kernel<MC, NCW, KSPLIT>), dim3(grid), dim3(kThreads), 0, s,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wg), bias, T,
                     H, E, k, idx, w, pp);
  return hipGetLastError();
}

template <int MC>
hipError_t launch_bf16_mc(const void* x, const void* wg, const float* bias, int T, int H, int E,
                          int k, int32_t* idx, float* w, float* pp, hipStream_t s) {
  const int nc = (E + 15) / 16;
  if (nc < 4) {
    switch (nc) {
      case 1: return launch_bf16<MC, 1, 4>(x, wg, bias, T, H, E, k, idx, w, pp, s);
      case 2: return launch_bf16<MC, 2, 4>(x, wg, bias, T, H, E, k, idx, w, pp, s);
      default: return launch_bf16<MC, 3, 4>(x, wg, bias, T, H, E, k, idx, w, pp, s);
    }
  }
  switch ((nc + 3) / 4) {
    case 1: return launch_bf16<MC, 1, 1>(x, wg, bias, T, H, E, k, idx, w, pp, s);
    case 2: return launch_bf16<MC, 2, 1>(x, wg, bias, T, H, E, k, idx, w, pp, s);
    case 3: return launch_bf16<MC, 3, 1>(x, wg, bias, T, H, E, k, idx, w, pp, s);
    default: return launch_bf16<MC, 4, 1>(x, wg, bias, T, H, E, k, idx, w, pp, s);
  }
}

// Tokens per workgroup of the one-launch bf16 path: as many as keep >= 256
// workgroups (one per CU).
int bf16_tokens_per_block(int T) { return T >= 64 * 256 ? 64 : T >= 32 * 256 ? 32 : 16; }

// Workgroups of the launch that runs the top-k (one partial probability row each).
int topk_blocks(int T, bool bf16) {
  if (route_two_phase(T, bf16)) return (T + 3) / 4;
  const int bt = bf16 ? bf16_tokens_per_block(T) : 16;
  return (T + bt - 1) / bt;
}

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

size_t scores_ws_bytes(int T, int H, int E, bool bf16) {
  if (!route_two_phase(T, bf16)) return 0;
  return align256((size_t)route_kslices(T, H, E) * T * E * sizeof(float));
}

}  // namespace

size_t route_ws_bytes(int T, int H, int E, bool bf16, bool prob) {
  size_t b = scores_ws_bytes(T, H, E, bf16);
  if (prob) b += align256((size_t)topk_blocks(T, bf16) * E * sizeof(float));
  return b;
}

hipError_t launch_route(const void* x, const void* wg, const float* bias, int T, int H, int E,
                        int k, bool bf16, int32_t* topk_idx, float* topk_w, float* prob_mean,
                        void* ws, hipStream_t s) {
  // partial probability sums sit after the partial score tiles
  float* pp = prob_mean == nullptr
                  ? nullptr
                  : reinterpret_cast<float*>(static_cast<char*>(ws) + scores_ws_bytes(T, H, E, bf16));
  hipError_t err = hipSuccess;
  if (route_two_phase(T, bf16)) {
    const int nks = route_kslices(T, H, E);
    const dim3 grid((T + 15) / 16, (E + 15) / 16, nks);
    hipLaunchKernelGGL(route_partial_kernel, grid, dim3(64), 0, s, static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(wg), T, H, E, (H / 32) / nks,
                       static_cast<float*>(ws));
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(route_select_kernel, dim3((T + 3) / 4), dim3(kThreads), 0, s,
                       static_cast<const float*>(ws), bias, T, E, k, nks, topk_idx, topk_w, pp);
    err = hipGetLastError();
  } else if (!bf16) {
    const int grid = (T + 15) / 16;
    hipLaunchKernelGGL(route_f32_kernel, dim3(grid), dim3(kThreads), 0, s,
                       static_cast<const float*>(x), static_cast<const float*>(wg), bias, T, H, E,
                       k, topk_idx, topk_w, pp);
    err = hipGetLastError();
  } else {
    switch (bf16_tokens_per_block(T)) {
      case 64: err = launch_bf16_mc<4>(x, wg, bias, T, H, E, k, topk_idx, topk_w, pp, s); break;
      case 32: err = launch_bf16_mc<2>(x, wg, bias, T, H, E, k, topk_idx, topk_w, pp, s); break;
      default: err = launch_bf16_mc<1>(x, wg, bias, T, H, E, k, topk_idx, topk_w, pp, s); break;
    }
  }
  if (err != hipSuccess || prob_mean == nullptr) return err;
  hipLaunchKernelGGL(prob_mean_kernel, dim3(1), dim3(kThreads), 0, s, pp, topk_blocks(T, bf16), T,
                     E, prob_mean);
  return hipGetLastError();
}

}  // namespace moe

// Step 5 - per-step load diagnostics from the expert counts.
//
// Method: "Kimi K3 专家路由不均衡诊断" section 3 (MoERouteDiagnostics):
//   capacity = int((T*k / E) * cf)             (double arithmetic, truncation)
//   overflow_e = max(0, c_e - capacity), dropped = sum overflow (counted only),
//   drop rate = dropped / (T*k), skew = max / (min + 1e-5),
//   Gini (sorted-index form) = 2*sum_i i*c_(i) / (n*sum c) - (n+1)/n, 0 if sum c = 0,
//   stragglers = ids with c_e > capacity.
// Gini is kept as the exact integer fraction (2*sum_i i*c_(i) - (n+1)*sum c) /
// (n*sum c) and rounded once by a double division. The ascending rank i of
// each count comes from comparisons (ties broken by id), which gives the
// same sum as sorting.
//
// One workgroup of 256 threads (E <= 256): thread e owns expert e.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

struct Stats {
  int64_t num_tokens, assignments, capacity, max_load, min_load, dropped, num_stragglers,
      gini_num, gini_den;
  double load_skew_ratio, gini, drop_rate;
};

// Sum, max and min over the 64 lanes of a wavefront through the partner<L>
// butterfly (DPP within 16 lanes, then a swizzle and a permute); exact
// integer arithmetic, so the pairing order does not matter.
template <int L = 0>
__device__ __forceinline__ long long wave_sum(long long v) {
  if constexpr (L < 6) return wave_sum<L + 1>(v + (long long)partner64<L>((uint64_t)v));
  return v;
}
template <int L = 0>
__device__ __forceinline__ int wave_max(int v) {
  if constexpr (L < 6) return wave_max<L + 1>(max(v, (int)partner<L>((uint32_t)v)));
  return v;
}
template <int L = 0>
__device__ __forceinline__ int wave_min(int v) {
  if constexpr (L < 6) return wave_min<L + 1>(min(v, (int)partner<L>((uint32_t)v)));
  return v;
}

__global__ __launch_bounds__(256) void stats_kernel(const int32_t* __restrict__ counts, int T,
                                                    int E, int k, double cf,
                                                    Stats* __restrict__ out,
                                                    int32_t* __restrict__ overflow,
                                                    int32_t* __restrict__ stragglers) {
  __shared__ __align__(16) int c[256];
  __shared__ __align__(16) uint32_t key[256];
  __shared__ long long w_sum[4], w_isum[4], w_drop[4];
  __shared__ int w_max[4], w_min[4], w_str[4];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  const long long assignments = (long long)T * k;
  const long long capacity = (long long)(((double)assignments / (double)E) * cf);
  const int ce = e < E ? counts[e] : 0;
  // With every count in [0, 2^24), (count << 8 | id) is a unique key whose
  // unsigned order is (count, id): one compare per pair. Padding keys are
  // never below a real one. Other counts take the plain comparisons.
  c[e] = ce;
  key[e] = e < E ? ((uint32_t)ce << 8) | (uint32_t)e : 0xFFFFFFFFu;
  const bool packed = !__syncthreads_or(e < E && (uint32_t)ce >= (1u << 24));
  long long rank = 0;  // 1-based ascending rank of c[e]
  int strag = 0;
  long long over = 0;
  if (e < E) {
    // 32 counts per round, all LDS reads issued before the comparisons
    int less = 0;
    if (packed) {
      const uint32_t mine = ((uint32_t)ce << 8) | (uint32_t)e;
      const uint4* k4 = reinterpret_cast<const uint4*>(key);
      for (int q0 = 0; q0 < E; q0 += 32) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = k4[q0 / 4 + u];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          less += (int)(v[u].x < mine) + (int)(v[u].y < mine) + (int)(v[u].z < mine) +
                  (int)(v[u].w < mine);
      }
    }
    const int4* c4 = reinterpret_cast<const int4*>(c);
    for (int q0 = 0; !packed && q0 < E; q0 += 32) {
      int4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = c4[q0 / 4 + u];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = q0 + 4 * u;
        less += (q + 0 < E) & ((v[u].x < ce) | ((v[u].x == ce) & (q + 0 < e)));
        less += (q + 1 < E) & ((v[u].y < ce) | ((v[u].y == ce) & (q + 1 < e)));
        less += (q + 2 < E) & ((v[u].z < ce) | ((v[u].z == ce) & (q + 2 < e)));
        less += (q + 3 < E) & ((v[u].w < ce) | ((v[u].w == ce) & (q + 3 < e)));
      }
    }
    rank = less + 1;
    over = ce > capacity ? ce - capacity : 0;
    strag = ce > capacity;
    if (overflow != nullptr) overflow[e] = (int32_t)over;
  }
  // per-wavefront totals, then the four wavefronts in LDS; the straggler
  // flags become positions in the ascending id list through a ballot
  const long long s_sum = wave_sum(ce);
  const long long s_isum = wave_sum(rank * ce);
  const long long s_drop = wave_sum(over);
  const int s_max = wave_max(e < E ? ce : INT_MIN);
  const int s_min = wave_min(e < E ? ce : INT_MAX);
  const unsigned long long smask = __ballot(strag);
  if (lane == 0) {
    w_sum[wave] = s_sum;
    w_isum[wave] = s_isum;
    w_drop[wave] = s_drop;
    w_max[wave] = s_max;
    w_min[wave] = s_min;
    w_str[wave] = __popcll(smask);
  }
  __syncthreads();
  int before = 0, nstrag = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) before += w_str[w];
    nstrag += w_str[w];
  }
  if (e < E) {
    if (strag) stragglers[before + __popcll(smask & ((1ull << lane) - 1))] = e;
    if (e >= nstrag) stragglers[e] = -1;
  }
  if (e == 0) {
    long long total = 0, isum = 0, dropped = 0;
    int mx = INT_MIN, mn = INT_MAX;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      total += w_sum[w];
      isum += w_isum[w];
      dropped += w_drop[w];
      mx = max(mx, w_max[w]);
      mn = min(mn, w_min[w]);
    }
    Stats s;
    s.num_tokens = T;
    s.assignments = assignments;
    s.capacity = capacity;
    s.max_load = mx;
    s.min_load = mn;
    s.dropped = dropped;
    s.num_stragglers = nstrag;
    if (total == 0) {
      s.gini_num = 0;
      s.gini_den = 1;
      s.gini = 0.0;
    } else {
      s.gini_num = 2 * isum - (long long)(E + 1) * total;
      s.gini_den = (long long)E * total;
      s.gini = (double)s.gini_num / (double)s.gini_den;
    }
    s.load_skew_ratio = (double)s.max_load / ((double)s.min_load + 1e-5);
    s.drop_rate = (double)dropped / (double)assignments;
    *out = s;
  }
}

}  // namespace

hipError_t launch_load_stats(const int32_t* counts, int T, int E, int k, double cf, void* stats,
                             int32_t* overflow, int32_t* straggler_ids, hipStream_t s) {
  hipLaunchKernelGGL(stats_kernel, dim3(1), dim3(256), 0, s, counts, T, E, k, cf,
                     static_cast<Stats*>(stats), overflow, straggler_ids);
  return hipGetLastError();
}

}  // namespace moe

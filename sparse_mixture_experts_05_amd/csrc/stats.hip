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

__global__ __launch_bounds__(256) void stats_kernel(const int32_t* __restrict__ counts, int T,
                                                    int E, int k, double cf,
                                                    Stats* __restrict__ out,
                                                    int32_t* __restrict__ overflow,
                                                    int32_t* __restrict__ stragglers) {
  __shared__ int c[256];
  __shared__ long long red_sum[256], red_isum[256], red_drop[256];
  __shared__ int red_max[256], red_min[256], red_str[256];
  const int e = threadIdx.x;
  const long long assignments = (long long)T * k;
  const long long capacity = (long long)(((double)assignments / (double)E) * cf);
  const int ce = e < E ? counts[e] : 0;
  c[e] = ce;
  __syncthreads();
  long long rank = 0;  // 1-based ascending rank of c[e]
  int strag = 0;
  long long over = 0;
  if (e < E) {
    int less = 0;
    for (int q = 0; q < E; ++q) less += (c[q] < ce) || (c[q] == ce && q < e);
    rank = less + 1;
    over = ce > capacity ? ce - capacity : 0;
    strag = ce > capacity;
    if (overflow != nullptr) overflow[e] = (int32_t)over;
  }
  red_sum[e] = ce;
  red_isum[e] = rank * ce;
  red_drop[e] = over;
  red_max[e] = e < E ? ce : INT_MIN;
  red_min[e] = e < E ? ce : INT_MAX;
  red_str[e] = strag;
  __syncthreads();
  // Inclusive scan of the straggler flags (for the ascending id list) and
  // tree reductions of the rest, 8 steps over 256 entries.
  for (int d = 1; d < 256; d <<= 1) {
    const int v = e >= d ? red_str[e - d] : 0;
    __syncthreads();
    red_str[e] += v;
    __syncthreads();
  }
  for (int d = 128; d > 0; d >>= 1) {
    if (e < d) {
      red_sum[e] += red_sum[e + d];
      red_isum[e] += red_isum[e + d];
      red_drop[e] += red_drop[e + d];
      red_max[e] = max(red_max[e], red_max[e + d]);
      red_min[e] = min(red_min[e], red_min[e + d]);
    }
    __syncthreads();
  }
  const int nstrag = red_str[255];
  if (e < E) {
    if (strag) stragglers[red_str[e] - 1] = e;
    if (e >= nstrag) stragglers[e] = -1;
  }
  if (e == 0) {
    const long long total = red_sum[0];
    const long long dropped = red_drop[0];
    Stats s;
    s.num_tokens = T;
    s.assignments = assignments;
    s.capacity = capacity;
    s.max_load = red_max[0];
    s.min_load = red_min[0];
    s.dropped = dropped;
    s.num_stragglers = nstrag;
    if (total == 0) {
      s.gini_num = 0;
      s.gini_den = 1;
      s.gini = 0.0;
    } else {
      s.gini_num = 2 * red_isum[0] - (long long)(E + 1) * total;
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

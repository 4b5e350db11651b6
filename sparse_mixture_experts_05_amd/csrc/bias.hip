// Dynamic routing bias and the load statistics of the balance term.
//
// Method: "Kimi K3 专家路由不均衡诊断" section 4.2: the router scores
// Softmax(Logits + B); a background monitor lowers B_i by a small step while
// expert i is overloaded and raises it while expert i is idle. Section 4.1
// names the statistic f_i (share of the routed tokens that expert i received).
//
// Overloaded means a count above the mean count sum(c)/E, idle one below it;
// the comparison c_e * E vs sum(c) is exact in 64-bit integers. The new bias
// is one fp32 addition or subtraction of gamma. f_e = c_e / sum(c) is divided
// in double and rounded once to fp32.
//
// One workgroup of 256 threads (E <= 256): thread e owns expert e.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ counts,
                                                          int E, float gamma,
                                                          float* __restrict__ bias,
                                                          float* __restrict__ frac) {
  __shared__ long long red[256];
  const int e = threadIdx.x;
  const long long c = e < E ? (long long)counts[e] : 0;
  red[e] = c;
  __syncthreads();
  for (int d = 128; d > 0; d >>= 1) {
    if (e < d) red[e] += red[e + d];
    __syncthreads();
  }
  const long long total = red[0];
  if (e < E) {
    const long long d = c * E - total;  // sign of c - mean
    float b = bias[e];
    if (d > 0) b = b - gamma;
    else if (d < 0) b = b + gamma;
    bias[e] = b;
    if (frac != nullptr) frac[e] = total > 0 ? (float)((double)c / (double)total) : 0.0f;
  }
}

}  // namespace

hipError_t launch_bias_update(const int32_t* counts, int E, float gamma, float* bias,
                              float* load_frac, hipStream_t s) {
  hipLaunchKernelGGL(bias_update_kernel, dim3(1), dim3(256), 0, s, counts, E, gamma, bias,
                     load_frac);
  return hipGetLastError();
}

}  // namespace moe

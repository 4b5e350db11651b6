// Step 2 - token dispatch: expert histogram, offsets, stable permutation and
// the gather of token rows into one expert-contiguous buffer.
//
// Method: "lpqz.cn MoE engineering blog" section 3.1 (the dispatcher groups
// token indices by expert id into one pre-allocated shared buffer, runs each
// expert on its group and scatters results back to the original order) and
// "Kimi K3 专家路由不均衡诊断" section 3 (per-expert hit counts). Here the buffer
// is unpadded: expert e owns rows [offsets[e], offsets[e+1]), filled in
// token order.
//
// Three launches (two when T <= 256: one block counts its own histogram),
// all deterministic (no order-dependent atomics):
//   hist    - one workgroup per block of bt tokens (64 for 256 < T <= 4096
//             and k >= 4, else 256): LDS-privatised histogram, written
//             expert-major as blk[e * nb + b].
//   rank    - one workgroup per block: every workgroup reads the whole
//             [E x nb] table (tiny, L2 resident) to get the expert offsets
//             (exclusive scan over experts) and its own prefix over earlier
//             blocks; then each wave walks its bt/4 tokens' assignments in order,
//             64 at a time, ranking equal expert ids with ballots (a lane's
//             rank = earlier lanes with the same id) on top of per-wave running
//             counters. Writes perm and inv (block 0 also counts and offsets).
//   scatter - one wavefront per token: reads the token's row once with 16-byte
//             loads and writes it to its k buffer rows.
// With a capacity cap >= 0 ("Kimi K3 专家路由不均衡诊断" section 3 counts the
// assignments past an expert's capacity, section 5 describes dropping them),
// an assignment whose rank among its expert's assignments (token order) is
// cap or more is dropped: inv = -1, no buffer row. offsets then describe the
// kept rows (min(count, cap) per expert); counts stay the raw counts.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

// Expert ids are in [0, E) by contract; clamping keeps a bad id from turning
// into an out-of-range position (hist and rank must agree, so both clamp).
__device__ __forceinline__ int expert_of(const int32_t* idx, int a, int E) {
  return min(max(idx[a], 0), E - 1);
}

constexpr int kThreads = 256;

// KP: k rounded up to a power of two (each thread holds KP ids); BT: tokens
// per block.
template <int KP, int BT>
__global__ __launch_bounds__(kThreads) void hist_kernel(const int32_t* __restrict__ idx, int T,
                                                        int E, int k, int nb,
                                                        int32_t* __restrict__ blk) {
  __shared__ int h[256];
  for (int e = threadIdx.x; e < E; e += kThreads) h[e] = 0;
  __syncthreads();
  const int a0 = blockIdx.x * BT * k;
  const int a1 = min(T, (blockIdx.x + 1) * BT) * k;
  // a1 - a0 <= kThreads * k: every id of the block is one of this thread's
  // KP, all loaded before the first count
  int ids[KP];
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const int a = a0 + threadIdx.x + kThreads * i;
    const int e = expert_of(idx, min(a, a1 - 1), E);  // unconditional load, in bounds
    ids[i] = a < a1 ? e : -1;
  }
#pragma unroll
  for (int i = 0; i < KP; ++i)
    if (ids[i] >= 0) atomicAdd(&h[ids[i]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) blk[(size_t)e * nb + blockIdx.x] = h[e];
}

template <int KP, int BT>
__global__ __launch_bounds__(kThreads) void rank_kernel(
    const int32_t* __restrict__ idx, int T, int E, int k, int nb, int cap,
    const int32_t* __restrict__ blk, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ int tot[256];      // per-expert kept totals, then inclusive scan
  __shared__ int koff[256];     // exclusive offsets of the kept rows
  __shared__ int run[4][256];   // per-wave running rank within the expert
  __shared__ int wcnt[4][256];  // per-wave counts
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;

  // Per-wave counts of this block (order-free integer adds).
  for (int w = 0; w < 4; ++w) wcnt[w][tid] = 0;
  __syncthreads();
  constexpr int wt = BT / 4;              // tokens per wave (at most 64)
  const int tw0 = b * BT + wave * wt;     // first token of this wave
  const int a0 = min(tw0, T) * k, a1 = min(tw0 + wt, T) * k;
  // a1 - a0 <= wt * k <= 64 * k: the wave's ids, KP per lane, all loaded up front
  // (row-major (t, j) order: id i of lane l is assignment a0 + 64 i + l)
  int ids[KP];
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const int a = a0 + lane + 64 * i;
    const int e = expert_of(idx, max(min(a, a1 - 1), 0), E);  // unconditional load, in bounds
    ids[i] = a < a1 ? e : -1;
  }
#pragma unroll
  for (int i = 0; i < KP; ++i)
    if (ids[i] >= 0) atomicAdd(&wcnt[wave][ids[i]], 1);
  __syncthreads();

  // Totals over all blocks and this block's prefix over earlier blocks. A
  // single block (nb == 1, launched without the histogram pass) has them in
  // its own wave counts.
  int total = 0, before = 0;
  if (tid < E) {
    if (nb == 1) {
      total = wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
    } else {
      // 16 loads of the row in flight at a time (exact integer sums)
      const int32_t* row = blk + (size_t)tid * nb;
      int i = 0;
      for (; i + 16 <= nb; i += 16) {
        int c[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) c[u] = row[i + u];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          total += c[u];
          if (i + u < b) before += c[u];
        }
      }
      for (; i < nb; ++i) {
        const int c = row[i];
        total += c;
        if (i < b) before += c;
      }
    }
  }
  const int kept = cap < 0 ? total : min(total, cap);
  tot[tid] = tid < E ? kept : 0;
  __syncthreads();
  // Exclusive scan of the kept totals over experts (Hillis-Steele on 256 entries).
  for (int d = 1; d < 256; d <<= 1) {
    const int v = tid >= d ? tot[tid - d] : 0;
    __syncthreads();
    tot[tid] += v;
    __syncthreads();
  }
  const int excl = tot[tid] - (tid < E ? kept : 0);
  koff[tid] = excl;
  if (b == 0 && tid < E) {
    counts[tid] = total;
    offsets[tid] = excl;
    if (tid == E - 1) offsets[E] = excl + kept;
  }

  if (tid < E) {
    int base = before;  // rank of this block's first assignment within the expert
    for (int w = 0; w < 4; ++w) {
      run[w][tid] = base;
      base += wcnt[w][tid];
    }
  }
  __syncthreads();

  // Stable ranking: assignments of this wave in row-major (t, j) order.
  int bits = 1;
  while ((1 << bits) < E + 1) ++bits;  // ids 0..E-1 plus the idle-lane id E
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const int c0 = a0 + 64 * i;
    if (c0 >= a1) break;
    const int a = c0 + lane;
    const bool valid = a < a1;
    const int e = valid ? ids[i] : E;
    uint64_t peers = ~0ull;
    for (int bt = 0; bt < bits; ++bt) {
      const uint64_t bal = __ballot((e >> bt) & 1);
      peers &= ((e >> bt) & 1) ? bal : ~bal;
    }
    const int rank = __popcll(peers & lt);
    int r = 0;
    if (valid) r = run[wave][e] + rank;  // rank within the expert, token order
    __builtin_amdgcn_wave_barrier();
    if (valid && rank == 0) run[wave][e] = r + __popcll(peers);
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      if (cap < 0 || r < cap) {
        const int pos = koff[e] + r;
        inv[a] = pos;
        perm[pos] = a;
      } else {
        inv[a] = -1;
      }
    }
  }
}

// One wavefront per token: read the row once, write it to its k buffer rows
// (dropped assignments, inv < 0, have none).
template <typename V>
__global__ __launch_bounds__(kThreads) void scatter_kernel(const V* __restrict__ x,
                                                           const int32_t* __restrict__ inv,
                                                           int T, int vec_per_row, int k,
                                                           V* __restrict__ xs) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kThreads / kWave) + (threadIdx.x >> 6);
  if (t >= T) return;
  // loads from indices clamped into the buffers (no branch and no wait per
  // load); the stores below skip the entries past k and past the row
  int dst[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) dst[j] = inv[(size_t)t * k + min(j, k - 1)];
  const V* src = x + (size_t)t * vec_per_row;
  for (int c = lane; c < vec_per_row; c += 4 * kWave) {
    V v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = src[min(c + u * kWave, vec_per_row - 1)];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        if (dst[j] >= 0) {
          V* d = xs + (size_t)dst[j] * vec_per_row;
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (c + u * kWave < vec_per_row) d[c + u * kWave] = v[u];
        }
      }
    }
  }
}

}  // namespace

// Tokens per hist/rank workgroup. Up to 256 tokens one workgroup does it all
// (no histogram launch). Up to 4096 tokens with k >= 4, 64-token blocks spread
// the ranking over up to 64 workgroups (each wave still ranks 64 or more ids).
// Otherwise 256-token blocks: they keep each wave's 64 lanes busy at small k,
// and keep short the [E x nb] table rows that every rank workgroup reads.
int dispatch_block_tokens(int T, int k) { return T > 256 && T <= 4096 && k >= 4 ? 64 : 256; }

template <int KP>
hipError_t launch_hist(const int32_t* idx, int T, int E, int k, int nb, int32_t* blk,
                       hipStream_t s) {
  if (dispatch_block_tokens(T, k) == 64)
    hipLaunchKernelGGL((hist_kernel<KP, 64>), dim3(nb), dim3(kThreads), 0, s, idx, T, E, k, nb, blk);
  else
    hipLaunchKernelGGL((hist_kernel<KP, 256>), dim3(nb), dim3(kThreads), 0, s, idx, T, E, k, nb, blk);
  return hipGetLastError();
}

template <int KP>
hipError_t launch_rank(const int32_t* idx, int T, int E, int k, int nb, int cap,
                       const int32_t* blk, int32_t* counts, int32_t* offsets, int32_t* perm,
                       int32_t* inv, hipStream_t s) {
  if (dispatch_block_tokens(T, k) == 64)
    hipLaunchKernelGGL((rank_kernel<KP, 64>), dim3(nb), dim3(kThreads), 0, s, idx, T, E, k, nb,
                       cap, blk, counts, offsets, perm, inv);
  else
    hipLaunchKernelGGL((rank_kernel<KP, 256>), dim3(nb), dim3(kThreads), 0, s, idx, T, E, k, nb,
                       cap, blk, counts, offsets, perm, inv);
  return hipGetLastError();
}

int dispatch_blocks(int T, int k) {
  const int bt = dispatch_block_tokens(T, k);
  return (T + bt - 1) / bt;
}

size_t dispatch_ws_bytes(int T, int E, int k) {
  const size_t b = (size_t)E * dispatch_blocks(T, k) * sizeof(int32_t);
  return (b + 255) & ~size_t(255);
}

hipError_t launch_dispatch(const int32_t* topk_idx, const void* x, int T, int H, int E, int k,
                           int cap, bool bf16, int32_t* counts, int32_t* offsets, int32_t* perm,
                           int32_t* inv, void* xs, void* ws, hipStream_t s) {
  const int nb = dispatch_blocks(T, k);
  int32_t* blk = static_cast<int32_t*>(ws);
  hipError_t err;
  if (nb > 1) {  // one block (T <= 256) counts its own histogram in the rank kernel
    err = k <= 1   ? launch_hist<1>(topk_idx, T, E, k, nb, blk, s)
          : k <= 2 ? launch_hist<2>(topk_idx, T, E, k, nb, blk, s)
          : k <= 4 ? launch_hist<4>(topk_idx, T, E, k, nb, blk, s)
                   : launch_hist<8>(topk_idx, T, E, k, nb, blk, s);
    if (err != hipSuccess) return err;
  }
  err = k <= 1   ? launch_rank<1>(topk_idx, T, E, k, nb, cap, blk, counts, offsets, perm, inv, s)
        : k <= 2 ? launch_rank<2>(topk_idx, T, E, k, nb, cap, blk, counts, offsets, perm, inv, s)
        : k <= 4 ? launch_rank<4>(topk_idx, T, E, k, nb, cap, blk, counts, offsets, perm, inv, s)
                 : launch_rank<8>(topk_idx, T, E, k, nb, cap, blk, counts, offsets, perm, inv, s);
  if (err != hipSuccess || xs == nullptr) return err;  // no xs: ranks only (gather fused downstream)
  const int row_bytes = H * (bf16 ? 2 : 4);
  const int grid = (T + 3) / 4;
  hipLaunchKernelGGL(scatter_kernel<uint4>, dim3(grid), dim3(kThreads), 0, s,
                     static_cast<const uint4*>(x), inv, T, row_bytes / 16, k,
                     static_cast<uint4*>(xs));
  return hipGetLastError();
}

// ----------------------------------------------------------------- no-alloc variant

namespace {

// Scratch of moe_dispatch_noalloc, for callers that cannot allocate: the
// [E x blocks] histogram table lives in this fixed device array instead of a
// caller workspace. Every GPU the library runs on holds its own copy until the
// process ends. Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, once per device.
constexpr size_t kNoAllocScratchBytes = size_t(1) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;

}  // namespace

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

// Device address of the current device's copy of `scratch`, looked up on the
// first call on that device (with it current) and kept per device.
hipError_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return hipSuccess;
}

// moe_dispatch on the fixed scratch: the same kernels, the table in `scratch`
// (its address from noalloc_scratch, never the array's name). Every entry of
// the table is written by the histogram launch before the rank launch reads
// it, so nothing needs clearing between calls. The caller has checked that
// dispatch_ws_bytes(T, E, k) fits kNoAllocScratchBytes.
hipError_t launch_dispatch_noalloc(const int32_t* topk_idx, const void* x, int T, int H, int E,
                                   int k, bool bf16, int32_t* counts, int32_t* offsets,
                                   int32_t* perm, int32_t* inv, void* xs, hipStream_t s) {
  if (dispatch_ws_bytes(T, E, k) > kNoAllocScratchBytes) return hipErrorInvalidValue;
  void* ws = nullptr;
  const hipError_t e = noalloc_scratch(&ws);
  if (e != hipSuccess) return e;
  return launch_dispatch(topk_idx, x, T, H, E, k, -1, bf16, counts, offsets, perm, inv, xs, ws, s);
}

}  // namespace moe

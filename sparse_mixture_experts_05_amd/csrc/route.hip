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
//            experts, K = H), fp32 accumulation, operands staged in LDS by
//            coalesced global -> LDS copies. fp32: plain dot products.
//   phase 2: the scores plus the bias go to an LDS tile; G = 256/BT lanes
//            per token each keep a sorted top-k list of 64-bit (score, id)
//            keys over a strided subset of the experts, merged across the G
//            lanes by bitonic merges over DPP / ds_swizzle / bpermute
//            exchanges. Ties go to the lower expert id.
// Few tokens (bf16, T < 2048, or T < 3072 when E > 128), and mid-size
// batches (T < 6144) with E > 64, take two launches: partial score tiles over
// K slices into the workspace, then a sum in slice order and the top-k.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxE = 256;

// Row stride (floats) of a score tile of BT tokens in a workgroup of NW
// waves. The top-k gives each token G = 64*NW/BT consecutive lanes; lane g of
// a token reads the columns g, g + G, ..., so a stride of G (mod 64) puts the
// 64 lanes of a wave on 64 distinct banks.
template <int BT, int NW = 4>
constexpr int tile_stride() { return kMaxE + NW * 64 / BT; }

// ---------------------------------------------------------------- top-k
// Every (score, expert) pair is one 64-bit key: the score's bits mapped to an
// order-preserving unsigned integer in the high half, the complement of the
// expert id in the low half. A larger key is a better entry: a higher score,
// or an equal score with a lower id. A NaN score reads as -inf and -0 as +0
// (they compare equal). Key 0 is below every real entry and marks an empty
// slot, so the k chosen ids are always real, distinct and < E.
// Written with arithmetic only (max with -inf drops a NaN, adding +0 turns
// -0 into +0, the sign mask flips the order of negatives): as selects the
// compiler turned the mapping into three nested branches per key.
__device__ __forceinline__ uint64_t topk_key(float s, int e) {
  const uint32_t u = __float_as_uint(fmaxf(s, -INFINITY) + 0.0f);
  const uint32_t o = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)(~(uint32_t)e);
}
__device__ __forceinline__ float key_score(uint64_t key) {
  const uint32_t o = (uint32_t)(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ int key_expert(uint64_t key) { return (int)(~(uint32_t)key); }

__device__ __forceinline__ void cswap(uint64_t& a, uint64_t& b) {  // a <- max, b <- min
  const bool gt = a > b;
  const uint64_t hi = gt ? a : b, lo = gt ? b : a;
  a = hi;
  b = lo;
}

// Sorts a bitonic sequence of N keys into descending order (half-cleaners).
template <int N>
__device__ __forceinline__ void bitonic_clean(uint64_t (&c)[N]) {
#pragma unroll
  for (int st = N / 2; st > 0; st >>= 1)
#pragma unroll
    for (int i = 0; i < N; ++i)
      if ((i & st) == 0) cswap(c[i], c[i + st]);
}

// Sorts N keys into descending order (bitonic sorting network).
template <int N>
__device__ __forceinline__ void bitonic_sort(uint64_t (&c)[N]) {
#pragma unroll
  for (int size = 2; size <= N; size <<= 1)
#pragma unroll
    for (int st = size / 2; st > 0; st >>= 1)
#pragma unroll
      for (int i = 0; i < N; ++i)
        if ((i & st) == 0) {
          if ((i & size) == 0) cswap(c[i], c[i + st]);
          else cswap(c[i + st], c[i]);
        }
}

// list <- the N largest of list and blk (both sorted descending): the
// elementwise max of list and reversed blk is bitonic and holds them.
template <int N>
__device__ __forceinline__ void merge_top(uint64_t (&list)[N], const uint64_t (&blk)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) list[i] = list[i] > blk[N - 1 - i] ? list[i] : blk[N - 1 - i];
  bitonic_clean<N>(list);
}

// Merge the lists of the G lanes of a token, levels 0 .. log2(G)-1; every
// lane ends with the same list.
template <int L, int G, int N>
__device__ __forceinline__ void group_merge(uint64_t (&list)[N]) {
  if constexpr ((1 << L) < G) {
    uint64_t other[N];
#pragma unroll
    for (int i = 0; i < N; ++i) other[i] = partner64<L>(list[i]);
    merge_top<N>(list, other);
    group_merge<L + 1, G, N>(list);
  }
}

// Sum over the G lanes of a token: each level adds a lane's value and its
// partner's, and fp addition is commutative, so every lane gets the same bits.
template <int L, int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr ((1 << L) < G) return group_sum<L + 1, G>(v + __uint_as_float(partner<L>(__float_as_uint(v))));
  return v;
}

// Top-k of the BT tokens whose scores (bias included) are in the LDS tile sc
// (row stride tile_stride<BT>()). Token t of the tile uses lanes
// [t*G, t*G + G); lane g reads the experts g, g + G, ... (at most EPX experts
// in all, a compile-time bound, so the scan is unrolled and branch free: all
// reads are issued first, from clamped columns, and columns >= E become
// empty keys), sorts blocks of KP keys and merges each into its running list,
// then the G lists are merged. KP >= k is a power of two.
// When pp is not null, the full softmax p[t, e] = exp(s_e - m) / sum_e' exp(s_e' - m)
// of every token overwrites its scores, and pp[e] receives the sum of p[t, e]
// over the tile's tokens (t ascending).
template <int BT, int KP, int EPX, int NW = 4>
__device__ __forceinline__ void topk_tokens(float* sc, int t0, int T, int E, int k,
                                            int32_t* __restrict__ topk_idx,
                                            float* __restrict__ topk_w, float* __restrict__ pp) {
  constexpr int NT = NW * 64;
  constexpr int G = NT / BT;
  constexpr int S = tile_stride<BT, NW>();
  static_assert(G >= 1 && G <= 64 && BT * G == NT, "one group of lanes per token");
  constexpr int NSUB = (EPX + G - 1) / G;  // experts per lane, at most
  constexpr int NBLK = (NSUB + KP - 1) / KP;
  const int t = threadIdx.x / G, g = threadIdx.x % G;
  const int tok = t0 + t;
  float* row = sc + t * S;
  const int nsub = (E + G - 1) / G;

  float v[NBLK * KP];
#pragma unroll
  for (int i = 0; i < NBLK * KP; ++i) v[i] = row[min(g + G * i, E - 1)];
  uint64_t list[KP];
#pragma unroll
  for (int b = 0; b < NBLK; ++b) {
    uint64_t blk[KP];
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const int e = g + G * (b * KP + i);
      // columns past E: an empty key (mask, not a select: see topk_key)
      blk[i] = topk_key(v[b * KP + i], e) & (uint64_t)(-(int64_t)(e < E));
    }
    bitonic_sort<KP>(blk);
    if (b == 0) {
#pragma unroll
      for (int i = 0; i < KP; ++i) list[i] = blk[i];
    } else {
      merge_top<KP>(list, blk);
    }
  }
  group_merge<0, G, KP>(list);

  // weights: exp(s_j - m) / sum over the k chosen, m = the best score
  const float m = key_score(list[0]);
  float ex[KP], sum = 0.0f;
#pragma unroll
  for (int j = 0; j < KP; ++j)
    if (j < k) {
      ex[j] = expf(key_score(list[j]) - m);
      sum += ex[j];
    }
  if (tok < T) {
#pragma unroll
    for (int j = 0; j < KP; ++j)
      if (j < k && j % G == g) {
        topk_idx[(size_t)tok * k + j] = key_expert(list[j]);
        topk_w[(size_t)tok * k + j] = ex[j] / sum;
      }
  }

  if (pp != nullptr) {
    // dead or NaN scores give 0; a token whose scores are all -inf or NaN has
    // no distribution and adds nothing
    float zs = 0.0f;
    for (int i = 0; i < nsub; ++i) {
      const int e = g + G * i;
      if (e < E) {
        const float v = row[e];
        const float z = (m > -INFINITY && v == v) ? expf(v - m) : 0.0f;
        row[e] = z;
        zs += z;
      }
    }
    const float Z = group_sum<0, G>(zs);
    for (int i = 0; i < nsub; ++i) {
      const int e = g + G * i;
      if (e < E) row[e] = Z > 0.0f ? row[e] / Z : 0.0f;
    }
    __syncthreads();
    const int nt = min(BT, T - t0);
    for (int e = threadIdx.x; e < E; e += NT) {
      float a = 0.0f;
      for (int q = 0; q < nt; ++q) a += sc[q * S + e];
      pp[e] = a;
    }
  }
}

template <int BT, int EPX, int NW = 4>
__device__ __forceinline__ void topk_phase(float* sc, int t0, int T, int E, int k,
                                           int32_t* __restrict__ topk_idx,
                                           float* __restrict__ topk_w, float* __restrict__ pp) {
  if (k <= 1) topk_tokens<BT, 1, EPX, NW>(sc, t0, T, E, k, topk_idx, topk_w, pp);
  else if (k <= 2) topk_tokens<BT, 2, EPX, NW>(sc, t0, T, E, k, topk_idx, topk_w, pp);
  else if (k <= 4) topk_tokens<BT, 4, EPX, NW>(sc, t0, T, E, k, topk_idx, topk_w, pp);
  else topk_tokens<BT, 8, EPX, NW>(sc, t0, T, E, k, topk_idx, topk_w, pp);
}

// P[e] = (sum over workgroups b, ascending, of part[b][e]) / T, in double.
__global__ __launch_bounds__(kThreads) void prob_mean_kernel(const float* __restrict__ part,
                                                             int nb, int T, int E,
                                                             float* __restrict__ prob_mean) {
  for (int e = threadIdx.x; e < E; e += kThreads) {
    double s = 0.0;
    int b = 0;
    for (; b + 16 <= nb; b += 16) {  // 16 loads in flight, then the sum in order
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = part[(size_t)(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < 16; ++u) s += (double)v[u];
    }
    for (; b < nb; ++b) s += (double)part[(size_t)b * E + e];
    prob_mean[e] = (float)(s / (double)T);
  }
}

// bf16 scores on MFMA 16x16x32 with operands staged in LDS. One workgroup
// (4 waves) computes a BT x EP tile of scores: BT tokens and EP experts
// starting at expert e0, over the K panels [kp0, kp1) of 64 elements.
// A panel holds the BT token rows, then the EP expert rows (R rows in all, a
// multiple of 32; rows past the data repeat a valid row and are never used),
// 128 bytes each. Rows are copied global -> LDS with global_load_lds: one
// instruction moves 8 rows, 8 consecutive lanes reading one whole 128-byte
// line. NS stages of PPS panels rotate through LDS, so two stages are in
// flight while one is multiplied. Chunk c (16 bytes) of LDS row r sits at
// slot c ^ ((r >> 1) & 7): a 128-bit read by 16 lanes (16 consecutive rows,
// one chunk) then touches 16 distinct 4-bank groups.
// Work split over the NW waves: EP >= 64, wave w computes experts
// [w*EP/NW, (w+1)*EP/NW) over all panels; EP < 64, wave w takes the panels
// p = w (mod NW) of every stage for the whole tile and the NW partial tiles
// are summed in wave order.
template <int BT, int EP, int NW = 4>
struct RouteTile {
  static constexpr int R = (BT + EP + 31) / 32 * 32;  // rows per panel
  static constexpr int PB = R * 128;                  // panel bytes
  static constexpr bool KSPLIT = EP < 64;
  static constexpr int PPS_RAW = (40 * 1024) / PB < 1 ? 1 : (40 * 1024) / PB;
  // panels per stage: a multiple of 4 when the waves split them, else <= 2
  static constexpr int PPS = KSPLIT ? (PPS_RAW >= 8 ? 8 : 4) : (PPS_RAW > 2 ? 2 : PPS_RAW);
  static constexpr int SB = PPS * PB;                 // stage bytes
  static constexpr int NS = 3;                        // stages
  static constexpr int NI = PPS * R / 8 / NW;         // DMA instructions per wave per stage
  static constexpr int MC = BT / 16;                  // 16-row tiles per wave
  static constexpr int NC = KSPLIT ? EP / 16 : EP / 16 / NW;  // 16-column tiles per wave
  static constexpr int SC_BYTES = BT * tile_stride<BT, NW>() * 4;
  static constexpr int PART_BYTES = KSPLIT ? NW * BT * EP * 4 : 0;
  static constexpr int LDS = NS * SB > SC_BYTES + PART_BYTES ? NS * SB : SC_BYTES + PART_BYTES;
  static_assert(PPS * R % (8 * NW) == 0, "whole DMA instructions per wave");
  static_assert(!KSPLIT || PPS % NW == 0, "the waves split each stage's panels evenly");
  static_assert(KSPLIT || NC >= 1, "whole 16-column tiles per wave");
  static_assert(NI < 32, "vmcnt range");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// The K loop of one tile; returns with every wave's accumulators complete and
// the LDS free for reuse (after a barrier).
template <int BT, int EP, int NW = 4>
__device__ __forceinline__ void score_tile(uint8_t* smem, const uint16_t* __restrict__ x,
                                           const uint16_t* __restrict__ wg, int t0, int T, int e0,
                                           int E, int H, int kp0, int kp1,
                                           f32x4_t (&acc)[RouteTile<BT, EP, NW>::MC][RouteTile<BT, EP, NW>::NC]) {
  using C = RouteTile<BT, EP, NW>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int NST = (kp1 - kp0 + C::PPS - 1) / C::PPS;  // stages

  // DMA plan of this lane: instruction q copies rows [8g, 8g+8) of panel pq[q].
  const uint16_t* src[C::NI];
  int pq[C::NI], dst[C::NI];
#pragma unroll
  for (int q = 0; q < C::NI; ++q) {
    const int j = wave * C::NI + q;
    const int p = j / (C::R / 8), g = j % (C::R / 8);
    const int r = 8 * g + (lane >> 3);
    const int chunk = (lane & 7) ^ ((r >> 1) & 7);
    const uint16_t* row = r < BT ? x + (size_t)min(t0 + r, T - 1) * H
                                 : wg + (size_t)min(e0 + r - BT, E - 1) * H;
    src[q] = row + chunk * 8;
    pq[q] = p;
    dst[q] = p * C::PB + g * 1024;
  }
  auto issue = [&](int st) {
    uint8_t* base = smem + (st % C::NS) * C::SB;
#pragma unroll
    for (int q = 0; q < C::NI; ++q)
      lds_dma16(src[q] + (size_t)min(kp0 + st * C::PPS + pq[q], kp1 - 1) * 64, base + dst[q]);
  };

#pragma unroll
  for (int m = 0; m < C::MC; ++m)
#pragma unroll
    for (int n = 0; n < C::NC; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // fragment of a 16-row tile: row lane%16, chunk ks*4 + lane/16 (a 32-deep k step)
  const int fr = (lane & 15) * 128;
  const int sw = (lane >> 1) & 7;
  const int c0 = C::KSPLIT ? 0 : wave * (EP / NW);

#pragma unroll
  for (int st = 0; st < C::NS - 1; ++st)
    if (st < NST) issue(st);
  for (int st = 0; st < NST; ++st) {
    if (st + C::NS - 2 < NST) wait_vmcnt<(C::NS - 2) * C::NI>();
    else wait_vmcnt<0>();
    lds_barrier();  // stage st landed for every wave; stage st-1 is no longer read
    if (st + C::NS - 1 < NST) issue(st + C::NS - 1);
    const uint8_t* base = smem + (st % C::NS) * C::SB;
#pragma unroll
    for (int p = 0; p < C::PPS; ++p) {
      if (C::KSPLIT && p % NW != wave) continue;
      if (kp0 + st * C::PPS + p >= kp1) continue;
      const uint8_t* pan = base + p * C::PB;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int slot = ((ks * 4 + (lane >> 4)) ^ sw) * 16;
        u32x4_t a[C::MC], b[C::NC];
#pragma unroll
        for (int m = 0; m < C::MC; ++m)
          a[m] = *reinterpret_cast<const u32x4_t*>(pan + m * 16 * 128 + fr + slot);
#pragma unroll
        for (int n = 0; n < C::NC; ++n)
          b[n] = *reinterpret_cast<const u32x4_t*>(pan + (BT + c0 + n * 16) * 128 + fr + slot);
#pragma unroll
        for (int m = 0; m < C::MC; ++m)
#pragma unroll
          for (int n = 0; n < C::NC; ++n)
            acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[m]), as_bf16x8(b[n]),
                                                                acc[m][n], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // every wave is done with the stages
}

// Scores of the tile plus the bias into LDS (row-major, tile_stride<BT>()),
// columns < ncol. D layout of 16x16: lane holds column lane%16, rows
// (lane/16)*4 + v.
template <int BT, int EP, int NW = 4>
__device__ __forceinline__ void scores_to_lds(uint8_t* smem, int ncol, const float* __restrict__ bias,
                                              const f32x4_t (&acc)[RouteTile<BT, EP, NW>::MC][RouteTile<BT, EP, NW>::NC]) {
  using C = RouteTile<BT, EP, NW>;
  constexpr int S = tile_stride<BT, NW>();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* sc = reinterpret_cast<float*>(smem);
  if (!C::KSPLIT) {
    const int c0 = wave * (EP / NW);
#pragma unroll
    for (int m = 0; m < C::MC; ++m)
#pragma unroll
      for (int n = 0; n < C::NC; ++n) {
        const int col = c0 + n * 16 + (lane & 15);
        const float b = (bias != nullptr && col < ncol) ? bias[col] : 0.0f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = m * 16 + (lane >> 4) * 4 + v;
          if (col < ncol) sc[row * S + col] = bias != nullptr ? acc[m][n][v] + b : acc[m][n][v];
        }
      }
  } else {
    float* part = reinterpret_cast<float*>(smem + C::SC_BYTES);
#pragma unroll
    for (int m = 0; m < C::MC; ++m)
#pragma unroll
      for (int n = 0; n < C::NC; ++n)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = m * 16 + (lane >> 4) * 4 + v;
          part[(wave * BT + row) * EP + n * 16 + (lane & 15)] = acc[m][n][v];
        }
    __syncthreads();
    for (int q = threadIdx.x; q < BT * ncol; q += NW * 64) {
      const int row = q / ncol, col = q % ncol;
      float v = part[(0 * BT + row) * EP + col];
#pragma unroll
      for (int w = 1; w < NW; ++w) v += part[(w * BT + row) * EP + col];  // waves in order
      sc[row * S + col] = bias != nullptr ? v + bias[col] : v;
    }
  }
  __syncthreads();
}

// One launch: BT tokens x all E experts (EP >= E) over all of H, then top-k,
// by NW waves.
template <int BT, int EP, int NW = 4>
__global__ __launch_bounds__(NW * 64) void route_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg,
    const float* __restrict__ bias, int T, int H, int E, int k, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ ppart) {
  using C = RouteTile<BT, EP, NW>;
  __shared__ __align__(16) uint8_t smem[C::LDS];
  const int t0 = blockIdx.x * BT;
  f32x4_t acc[C::MC][C::NC];
  score_tile<BT, EP, NW>(smem, x, wg, t0, T, 0, E, H, 0, H / 64, acc);
  scores_to_lds<BT, EP, NW>(smem, E, bias, acc);
  topk_phase<BT, EP, NW>(reinterpret_cast<float*>(smem), t0, T, E, k, topk_idx, topk_w,
                         ppart != nullptr ? ppart + (size_t)blockIdx.x * E : nullptr);
}

// fp32 scores with plain dot products (small fp32 layers).
__global__ __launch_bounds__(kThreads) void route_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wg, const float* __restrict__ bias,
    int T, int H, int E, int k, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ ppart) {
  constexpr int BT = 16;
  constexpr int S = tile_stride<BT>();
  __shared__ float sc[BT * S];
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
    sc[t * S + e] = bias != nullptr ? s + bias[e] : s;
  }
  __syncthreads();
  topk_phase<BT, kMaxE>(sc, t0, T, E, k, topk_idx, topk_w,
                        ppart != nullptr ? ppart + (size_t)blockIdx.x * E : nullptr);
}


// Two launches (bf16). Phase 1: workgroup (token block, expert block, K slice)
// computes its BT x EP partial score tile and stores it in the workspace
// ws[ks][t][e]. Phase 2: a workgroup of 4 or 16 tokens sums each token's K
// slices in a fixed order (ks ascending), adds the bias and runs the top-k.
//   Few tokens: 16 x 64 tiles, so that a few tokens still spread Wg over
//   about 256 workgroups (one workgroup per 16 tokens would stream all of Wg
//   through a single CU).
//   Mid-size batches and E > 64: 64 x 128 (E <= 128) or 128 x 256 tiles, so
//   that Wg is read once per 64 or 128 tokens instead of once per 16-64, the
//   L2 -> LDS traffic that bounds the one-launch kernel at large E.
constexpr int kPartBT = 16, kPartEP = 64, kMaxSlices = 16;

template <int BT, int EP, int NW = 4>
__global__ __launch_bounds__(NW * 64) void route_partial_kernel(const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ wg,
                                                                int T, int H, int E, int kps,
                                                                float* __restrict__ ws) {
  using C = RouteTile<BT, EP, NW>;
  static_assert(!C::KSPLIT, "each wave owns EP / NW experts");
  __shared__ __align__(16) uint8_t smem[C::NS * C::SB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * BT, e0 = blockIdx.y * EP, ks = blockIdx.z;
  f32x4_t acc[C::MC][C::NC];
  score_tile<BT, EP, NW>(smem, x, wg, t0, T, e0, E, H, ks * kps, (ks + 1) * kps, acc);
  // D layout of 16x16: lane holds column lane%16, rows (lane/16)*4 + v
#pragma unroll
  for (int m = 0; m < C::MC; ++m)
#pragma unroll
    for (int n = 0; n < C::NC; ++n) {
      const int e = e0 + wave * (EP / NW) + n * 16 + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = t0 + m * 16 + (lane >> 4) * 4 + v;
        if (t < T && e < E) ws[((size_t)ks * T + t) * E + e] = acc[m][n][v];
      }
    }
}

// BT tokens per workgroup: 256 / BT lanes per token in the top-k. Few lanes
// per token sort whole blocks of experts and merge over fewer levels; many
// lanes per token keep small batches spread over more workgroups.
template <int NKS, int BT, int EPX>
__global__ __launch_bounds__(kThreads) void route_select_kernel(const float* __restrict__ ws,
                                                                const float* __restrict__ bias,
                                                                int T, int E, int k,
                                                                int32_t* __restrict__ topk_idx,
                                                                float* __restrict__ topk_w,
                                                                float* __restrict__ ppart) {
  constexpr int S = tile_stride<BT>();
  __shared__ float sc[BT * S];
  const int t0 = blockIdx.x * BT;
  // PER entries per thread at a time (about 32 loads in flight): all their
  // slice loads are issued first, from addresses clamped into the buffer, then
  // each entry is summed in slice order
  constexpr int PER = NKS >= 8 ? 32 / NKS : 8;
  const int nval = min(BT, T - t0) * E;  // entries of the tile's real tokens (t-major)
  for (int p0 = threadIdx.x; p0 < nval; p0 += PER * kThreads) {
    float v[PER][NKS], bv[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int p = p0 + i * kThreads;
      const int tt = min(t0 + p / E, T - 1), e = p % E;
#pragma unroll
      for (int q = 0; q < NKS; ++q) v[i][q] = ws[((size_t)q * T + tt) * E + e];
      bv[i] = bias != nullptr ? bias[e] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int p = p0 + i * kThreads;
      const int t = p / E, e = p % E;
      if (p < nval) {
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < NKS; ++q) s += v[i][q];
        sc[t * S + e] = bias != nullptr ? s + bv[i] : s;
      }
    }
  }
  __syncthreads();
  topk_phase<BT, EPX>(sc, t0, T, E, k, topk_idx, topk_w,
                      ppart != nullptr ? ppart + (size_t)blockIdx.x * E : nullptr);
}

// The select for exactly nks K slices (a power of two up to kMaxSlices) and
// at most EPX experts.
template <int BT, int EPX>
hipError_t launch_select_e(int nks, const float* ws, const float* bias, int T, int E, int k,
                           int32_t* idx, float* w, float* pp, hipStream_t s) {
  const dim3 grid((T + BT - 1) / BT), block(kThreads);
  switch (nks) {
    case 1: hipLaunchKernelGGL((route_select_kernel<1, BT, EPX>), grid, block, 0, s, ws, bias, T, E, k, idx, w, pp); break;
    case 2: hipLaunchKernelGGL((route_select_kernel<2, BT, EPX>), grid, block, 0, s, ws, bias, T, E, k, idx, w, pp); break;
    case 4: hipLaunchKernelGGL((route_select_kernel<4, BT, EPX>), grid, block, 0, s, ws, bias, T, E, k, idx, w, pp); break;
    case 8: hipLaunchKernelGGL((route_select_kernel<8, BT, EPX>), grid, block, 0, s, ws, bias, T, E, k, idx, w, pp); break;
    case 16: hipLaunchKernelGGL((route_select_kernel<16, BT, EPX>), grid, block, 0, s, ws, bias, T, E, k, idx, w, pp); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BT>
hipError_t launch_select(int nks, const float* ws, const float* bias, int T, int E, int k,
                         int32_t* idx, float* w, float* pp, hipStream_t s) {
  if (E <= 64) return launch_select_e<BT, 64>(nks, ws, bias, T, E, k, idx, w, pp, s);
  if (E <= 128) return launch_select_e<BT, 128>(nks, ws, bias, T, E, k, idx, w, pp, s);
  return launch_select_e<BT, kMaxE>(nks, ws, bias, T, E, k, idx, w, pp, s);
}

// Path of a route call. Both two-launch paths write and re-read T x E partial
// scores per K slice, so their time grows faster with T than the one-launch
// path's; the one-launch path re-reads Wg once per 16, 32 or 64 tokens.
// Measured crossovers (H = 4096, k = 8): small tiles against one launch near
// T = 2048 up to E = 128 and near 3072 for E = 256 (graph replay, 4-wave
// tiles); small against big tiles near T = 2048 (E = 128: 18.0 against 18.5
// us at 1024, equal at 2048; E = 256: 26.7 against 27.8 at 1024, 35.0
// against 31.0 at 2048; route alone, read-flushed caches). Big tiles
// against one launch (route alone, read-flushed caches, 8-wave tiles on both
// paths for E >= 128): E = 128 30.0 against 54.7 us at T = 6144, 32.4
// against 33.3 at 8192, 47.5 against 58.9 at 12288, 45.9 against 46.1 at
// 16384; E = 256 39.3 against 85.8 at 6144, 59.6 against 99.3 at 12288,
// 62.9 against 63.1 at 16384. So big tiles up to T = 16384, where the
// one-launch path has 64-token tiles.

// Waves of a workgroup of the bf16 score kernels: 8 for tiles of 128 or more
// experts whose panels split into whole copy instructions over 8 waves, else
// 4. With 8, a CU keeps twice the waves issuing the L2 -> LDS copies of Wg
// (the same bytes in flight stream faster: a microbenchmark read 75 against
// 49 GB/s per CU with 32 KiB in flight) and the top-k has twice the lanes per
// token.
template <int BT, int EP>
constexpr int route_waves() {
  using C = RouteTile<BT, EP>;  // its panel rows and panels per stage do not depend on the waves
  // panel-split tiles (E <= 32) stay at 4: with 8 (one panel of each stage per
  // wave) the Mixtral-shaped route took 12.4 against 12.0 us
  if (C::KSPLIT) return 4;
  return EP >= 128 && (C::PPS * C::R) % 64 == 0 ? 8 : 4;
}

enum RouteMode { kOneLaunch, kTwoSmall, kTwoBig };
RouteMode route_mode(int T, int E, bool bf16) {
  if (!bf16) return kOneLaunch;
  if (T < 2048) return kTwoSmall;
  return E > 64 && T < 16384 ? kTwoBig : kOneLaunch;
}
bool route_two_phase(int T, int E, bool bf16) { return route_mode(T, E, bf16) != kOneLaunch; }

// Tile of the big-tile path.
int big_bt(int E) { return E > 128 ? 128 : 64; }
int big_ep(int E) { return E > 128 ? 256 : 128; }

// K slices of a two-launch path: about 256 workgroups in phase 1, a power of
// two (at most kMaxSlices) that divides the H/64 panels.
int route_kslices(int T, int H, int E) {
  const bool big = route_mode(T, E, true) == kTwoBig;
  const int bt = big ? big_bt(E) : kPartBT, ep = big ? big_ep(E) : kPartEP;
  const int tiles = ((T + bt - 1) / bt) * ((E + ep - 1) / ep);
  int ks = 1;
  while (ks * 2 * tiles <= 256 && (H / 64) % (ks * 2) == 0 && ks * 2 <= kMaxSlices) ks *= 2;
  return ks;
}

template <int BT, int EP, int NW = 4>
hipError_t launch_bf16(const void* x, const void* wg, const float* bias, int T, int H, int E,
                       int k, int32_t* idx, float* w, float* pp, hipStream_t s) {
  const int grid = (T + BT - 1) / BT;
  hipLaunchKernelGGL((route_bf16_kernel<BT, EP, NW>), dim3(grid), dim3(NW * 64), 0, s,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wg), bias, T,
                     H, E, k, idx, w, pp);
  return hipGetLastError();
}

template <int BT>
hipError_t launch_bf16_bt(const void* x, const void* wg, const float* bias, int T, int H, int E,
                          int k, int32_t* idx, float* w, float* pp, hipStream_t s) {
  if (E <= 16) return launch_bf16<BT, 16>(x, wg, bias, T, H, E, k, idx, w, pp, s);
  if (E <= 32) return launch_bf16<BT, 32>(x, wg, bias, T, H, E, k, idx, w, pp, s);
  if (E <= 64) return launch_bf16<BT, 64>(x, wg, bias, T, H, E, k, idx, w, pp, s);
  if (E <= 128) return launch_bf16<BT, 128, route_waves<BT, 128>()>(x, wg, bias, T, H, E, k, idx, w, pp, s);
  return launch_bf16<BT, 256, route_waves<BT, 256>()>(x, wg, bias, T, H, E, k, idx, w, pp, s);
}

// Tokens per workgroup of the one-launch bf16 path: as many as keep >= 256
// workgroups (one per CU).
int bf16_tokens_per_block(int T) { return T >= 64 * 256 ? 64 : T >= 32 * 256 ? 32 : 16; }

// Tokens per workgroup of the two-launch select: 16 from T = 1024 up (at
// least 64 workgroups), else 4. Measured on the whole route of the
// fine-grained layer (T = 4096, H = 4096, E = 128, k = 8): 34.5 -> 33.2 us.
// Up to 4 tokens there is one workgroup either way, and 16 lanes per token
// merge over fewer levels than 64.
int select_tokens_per_block(int T) { return T >= 1024 || T <= 4 ? 16 : 4; }

// Workgroups of the launch that runs the top-k (one partial probability row each).
int topk_blocks(int T, int E, bool bf16) {
  if (route_two_phase(T, E, bf16)) {
    const int bt = select_tokens_per_block(T);
    return (T + bt - 1) / bt;
  }
  const int bt = bf16 ? bf16_tokens_per_block(T) : 16;
  return (T + bt - 1) / bt;
}

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

size_t scores_ws_bytes(int T, int H, int E, bool bf16) {
  if (!route_two_phase(T, E, bf16)) return 0;
  return align256((size_t)route_kslices(T, H, E) * T * E * sizeof(float));
}

}  // namespace

size_t route_ws_bytes(int T, int H, int E, bool bf16, bool prob) {
  size_t b = scores_ws_bytes(T, H, E, bf16);
  if (prob) b += align256((size_t)topk_blocks(T, E, bf16) * E * sizeof(float));
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
  const RouteMode mode = route_mode(T, E, bf16);
  if (mode != kOneLaunch) {
    const int nks = route_kslices(T, H, E);
    const int kps = (H / 64) / nks;
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    const uint16_t* wp = static_cast<const uint16_t*>(wg);
    float* sp = static_cast<float*>(ws);
    if (mode == kTwoSmall) {
      const dim3 grid((T + kPartBT - 1) / kPartBT, (E + kPartEP - 1) / kPartEP, nks);
      hipLaunchKernelGGL((route_partial_kernel<kPartBT, kPartEP>), grid, dim3(kThreads), 0, s, xp,
                         wp, T, H, E, kps, sp);
    } else if (E > 128) {
      const dim3 grid((T + 127) / 128, (E + 255) / 256, nks);
      hipLaunchKernelGGL((route_partial_kernel<128, 256, route_waves<128, 256>()>), grid,
                         dim3(route_waves<128, 256>() * 64), 0, s, xp, wp, T,
                         H, E, kps, sp);
    } else {
      const dim3 grid((T + 63) / 64, (E + 127) / 128, nks);
      hipLaunchKernelGGL((route_partial_kernel<64, 128, route_waves<64, 128>()>), grid,
                         dim3(route_waves<64, 128>() * 64), 0, s, xp, wp, T, H,
                         E, kps, sp);
    }
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const float* wsf = static_cast<const float*>(ws);
    err = select_tokens_per_block(T) == 16
              ? launch_select<16>(nks, wsf, bias, T, E, k, topk_idx, topk_w, pp, s)
              : launch_select<4>(nks, wsf, bias, T, E, k, topk_idx, topk_w, pp, s);
  } else if (!bf16) {
    const int grid = (T + 15) / 16;
    hipLaunchKernelGGL(route_f32_kernel, dim3(grid), dim3(kThreads), 0, s,
                       static_cast<const float*>(x), static_cast<const float*>(wg), bias, T, H, E,
                       k, topk_idx, topk_w, pp);
    err = hipGetLastError();
  } else {
    switch (bf16_tokens_per_block(T)) {
      case 64: err = launch_bf16_bt<64>(x, wg, bias, T, H, E, k, topk_idx, topk_w, pp, s); break;
      case 32: err = launch_bf16_bt<32>(x, wg, bias, T, H, E, k, topk_idx, topk_w, pp, s); break;
      default: err = launch_bf16_bt<16>(x, wg, bias, T, H, E, k, topk_idx, topk_w, pp, s); break;
    }
  }
  if (err != hipSuccess || prob_mean == nullptr) return err;
  hipLaunchKernelGGL(prob_mean_kernel, dim3(1), dim3(kThreads), 0, s, pp, topk_blocks(T, E, bf16), T,
                     E, prob_mean);
  return hipGetLastError();
}

}  // namespace moe

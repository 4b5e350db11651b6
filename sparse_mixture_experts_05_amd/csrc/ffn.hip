// Step 3 - grouped expert FFN over the expert-contiguous buffer.
//
// Method: "lpqz.cn MoE engineering blog" section 3.1 (each expert is two
// Linear layers with a GeLU between them) and the "hncyxsy.com Kimi K3
// fine-grained MoE" article (top-8 of many small experts plus one always-on
// shared expert; FFN cost 2*B*S*K*(2*H*D_ffn) FLOPs).
//
// Two launches of one grouped-GEMM kernel:
//   up:   h[p, :]  = GeLU(xs[p, :] . W1[e]^T)   N = F,  K = H  (erf-GeLU epilogue)
//   down: ys[p, :] = h[p, :] . W2[e]^T           N = H,  K = F
// Each launch also carries the shared expert as one more group (x -> hs -> ysh).
//
// Tiles: a workgroup covers rows [row0, row0+BM) of one expert segment and
// columns [n0, n0+BN). The expert of a tile is looked up on the device from
// offsets, so the host never reads the routing: the small-tile kernels scan
// per-expert tile counts in LDS; the big-tile launches read a tile table that
// one planning launch (big_plan_kernel) writes for both GEMMs. The grid is
// sized for the worst case (sum over experts of ceil(count/BM) <= rows/BM +
// min(E, rows)); surplus workgroups exit at once.
//
// bf16 kernels (fp32 accumulation). The tile kernels copy operands global ->
// LDS with global_load_lds (8 rows of 128 contiguous bytes per instruction),
// 16-byte chunks XOR-swizzled by row so fragment reads are bank-conflict free,
// and multiply with v_mfma_f32_32x32x16_bf16; rows past the segment end are
// clamped on load and masked on store:
//   gemm_bf16_w4_kernel    256x256 tiles, 4 waves (one per SIMD), 2 A and 3 B
//                          LDS stages, blocked XCD-aware tile order, split K
//                          in the last round of long-K launches
//                          (gemm_tail_reduce_kernel sums it);
//   gemm_bf16_big_kernel   the same tiles on 8 waves with 64-bit row offsets
//                          (an operand buffer of 4 GiB or more); segments of
//                          at most 32 rows as pairs of 32x128 tiles;
//   gemm_bf16_kernel       32x64 tiles for launches with few rows per expert:
//                          weight streaming through a 3-stage ring, split over
//                          K when there are fewer tiles than CUs
//                          (gemm_small_reduce_kernel sums the slices);
//   gemm_bf16_rows_kernel  decode launches (up to about two rows per expert):
//                          16-row blocks, weights loaded straight to registers
//                          and multiplied with v_mfma_f32_16x16x32_bf16, K
//                          split over the waves of a workgroup.
// fp32 path (small fp32 layers): 64x64 tiles of plain FMA.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "common.hpp"
#include "kernels.hpp"
#include "plan.hpp"


namespace moe {
namespace {

constexpr int kThreads = 256;

struct Group {
  const void* A;  // [M, K] rows (routed: the whole buffer; shared: x or hs)
  const void* B;  // routed: [E, N, K]; shared: [N, K]
  void* C;        // [M, N]
  int N, K;
};

struct GemmArgs {
  Group routed, shared;
  const int32_t* offsets;  // [E+1]
  int E;
  int rows;          // rows of the routed buffer
  int routed_tiles;  // grid share of the routed group: mtiles_max * ntiles
  int shared_M;      // 0 = no shared group
  int gelu;
  float* part;       // split-K partial tiles of the last round (big kernel), or null
  const int4* table; // big kernel: tile descriptors, 2 per slot (launch slots, then reduce slots)
  int slots;         // big kernel: workgroups of the launch (= reduce table start)
  const int32_t* gather;  // routed rows read through perm: A row p = token perm[p] / gk, or null
  int gk, gT;             // experts per token and tokens of that gather
  int wide;               // an A operand buffer of 4 GiB or more: the 8-wave kernel
                          // (which alone takes short segments as tile pairs)
};

// Row of the A operand that buffer row p of a group reads: p itself, or for
// the routed group of a gathering launch the token perm[p] / k (perm clamped
// into [0, T*k), so no read leaves x).
__device__ __forceinline__ size_t a_row(const GemmArgs& a, int group, int p) {
  if (group == 0 && a.gather != nullptr) {
    const int v = min(max(a.gather[p], 0), a.gT * a.gk - 1);
    return (size_t)(v / a.gk);
  }
  return (size_t)p;
}

using plan::Tile;

// f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N-1>{}):
// a loop whose index is a compile-time constant in every step, so register
// arrays indexed by it stay in registers.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Field-wise select (a reference into the kernel arguments chosen at run time
// would force a private-memory copy of the whole struct).
__device__ __forceinline__ Group pick_group(const GemmArgs& a, int group) {
  Group g;
  g.A = group ? a.shared.A : a.routed.A;
  g.B = group ? a.shared.B : a.routed.B;
  g.C = group ? a.shared.C : a.routed.C;
  g.N = group ? a.shared.N : a.routed.N;
  g.K = group ? a.shared.K : a.routed.K;
  return g;
}

// Finds the tile of this workgroup. Returns false if it has no work.
template <int BM, int BN>
__device__ bool find_tile(const GemmArgs& a, Tile& t) {
  __shared__ int pre[256];
  __shared__ int sel[3];
  const int g = blockIdx.x;
  if (g >= a.routed_tiles) {
    const int gs = g - a.routed_tiles;
    const int ntn = (a.shared.N + BN - 1) / BN;
    t.group = 1;
    t.e = 0;
    t.row0 = (gs / ntn) * BM;
    t.M = min(BM, a.shared_M - t.row0);
    t.n0 = (gs % ntn) * BN;
    return t.M > 0;
  }
  const int ntn = (a.routed.N + BN - 1) / BN;
  const int mt = g / ntn;
  const int tid = threadIdx.x;
  int off = 0, cnt = 0, tiles = 0;
  if (tid < a.E) {
    // offsets come from the dispatch step; clamping keeps any segment inside
    // the buffer even if a caller passes inconsistent offsets
    off = min(max(a.offsets[tid], 0), a.rows);
    cnt = min(max(a.offsets[tid + 1], off), a.rows) - off;
    tiles = (cnt + BM - 1) / BM;
  }
  pre[tid] = tiles;
  if (tid == 0) sel[0] = -1;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    const int v = tid >= d ? pre[tid - d] : 0;
    __syncthreads();
    pre[tid] += v;
    __syncthreads();
  }
  if (tid < a.E) {
    const int incl = pre[tid], excl = incl - tiles;
    if (mt >= excl && mt < incl) {
      sel[0] = tid;
      sel[1] = off + (mt - excl) * BM;
      sel[2] = min(BM, cnt - (mt - excl) * BM);
    }
  }
  __syncthreads();
  t.group = 0;
  t.e = sel[0];
  t.row0 = sel[1];
  t.M = sel[2];
  t.n0 = (g % ntn) * BN;
  return t.e >= 0;
}

// The big-tile schedule (tile order, split-K last round, short-segment
// pairs) is plain integer arithmetic in plan.hpp, shared with host checks.
using plan::kBlockCols;
using plan::kMaxSplit;
using plan::kReduceSlots;
using plan::kSBM;
using plan::kSBN;
using plan::kSlots;
using plan::kXcds;
constexpr int kBigWaves = 8;
constexpr size_t kPartTiles = (size_t)kXcds * kSlots;  // split units at most
constexpr int kTableInt4 = plan::kEntryInts / 4;       // int4 per table entry

__device__ __forceinline__ plan::Shape shape_of(const GemmArgs& a) {
  return plan::Shape{a.E,         a.rows,      a.shared_M,
                     a.routed.N,  a.routed.K,  a.shared.N,
                     a.shared.K,  a.part != nullptr ? 1 : 0, a.slots, a.wide};
}

// The schedule of a big-tile launch, computed by every workgroup of the
// planning launch: thread g fills the table entries of group g (thread 255
// also carries group 256, the shared expert next to 256 routed experts), the
// tables are scanned in LDS, and plan::finish_schedule derives the rest.
template <int BM, int BN>
__device__ plan::Sched big_schedule(const plan::Shape& sh, const int32_t* offsets,
                                    plan::Tables& L) {
  // Only the first 256 threads take part (the workgroup may be larger);
  // every thread still meets every barrier.
  const int tid = threadIdx.x;
  const bool act = tid < 256;
  int off = 0, cnt = 0, all = 0, big = 0, sml = 0;
  if (act) plan::group_entry<BM, BN>(sh, offsets, tid, off, cnt, all, big, sml);
  int o2 = 0, c2 = 0, all2 = 0, big2 = 0, sml2 = 0;
  if (tid == 255) plan::group_entry<BM, BN>(sh, offsets, 256, o2, c2, all2, big2, sml2);
  if (act) {
    L.goff[tid] = off;
    L.gcnt[tid] = cnt;
    L.pa[tid] = all;
    L.pf[tid] = big;
    L.ps[tid] = sml;
  }
  if (tid == 255) {
    L.goff[256] = o2;
    L.gcnt[256] = c2;
  }
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    const int va = (act && tid >= d) ? L.pa[tid - d] : 0;
    const int vf = (act && tid >= d) ? L.pf[tid - d] : 0;
    const int vs = (act && tid >= d) ? L.ps[tid - d] : 0;
    __syncthreads();
    if (act) {
      L.pa[tid] += va;
      L.pf[tid] += vf;
      L.ps[tid] += vs;
    }
    __syncthreads();
  }
  if (tid == 255) {
    L.pa[256] = L.pa[255] + all2;
    L.pf[256] = L.pf[255] + big2;
    L.ps[256] = L.ps[255] + sml2;
  }
  __syncthreads();
  return plan::finish_schedule(sh, L);
}

// Writes the tile table of one big-tile launch (plan::encode_entry, four int4
// per workgroup slot): slots [0, a.slots) for the GEMM launch (workgroup g:
// slot g / 8 on XCD g % 8), then kReduceSlots for its split-K reduce. Every
// workgroup computes the same schedule (group scans, from offsets), then each
// thread resolves one slot: the GEMM workgroups read one entry instead of each
// redoing the schedule.
template <int BM, int BN, int GN>
__device__ void plan_launch(const GemmArgs& a, int4* table, plan::Tables& L) {
  const plan::Shape sh = shape_of(a);
  const plan::Sched S = big_schedule<BM, BN>(sh, a.offsets, L);
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= a.slots + kReduceSlots) return;
  const int mode = i < a.slots ? 0 : 1;
  const int g = mode ? i - a.slots : i;
  Tile ta{}, tb{};
  const int kind = plan::resolve_slot<BM, BN, GN>(sh, S, L, g % kXcds, g / kXcds, mode, ta, tb);
  int e[plan::kEntryInts];
  plan::encode_entry(kind, ta, tb, e);
  int4* dst = table + kTableInt4 * i;
#pragma unroll
  for (int q = 0; q < kTableInt4; ++q)
    dst[q] = make_int4(e[4 * q], e[4 * q + 1], e[4 * q + 2], e[4 * q + 3]);
}

// One launch plans both GEMMs of the FFN (blockIdx.y: 0 up, 1 down).
template <int BM, int BN, int GN>
__global__ __launch_bounds__(kThreads) void big_plan_kernel(GemmArgs up, GemmArgs down) {
  __shared__ plan::Tables L;
  if (blockIdx.y == 0)
    plan_launch<BM, BN, GN>(up, const_cast<int4*>(up.table), L);
  else
    plan_launch<BM, BN, GN>(down, const_cast<int4*>(down.table), L);
}

// The work of table entry i (written by big_plan_kernel): returns its kind.
__device__ __forceinline__ int table_entry(const GemmArgs& a, int i, Tile& ta, Tile& tb) {
  const int4* e = a.table + kTableInt4 * i;
  const int4 d0 = e[0];
  if (d0.x < 0) return -1;
  const int4 d1 = e[1], d2 = e[2], d3 = e[3];
  ta.group = d0.y;
  ta.e = d0.z;
  ta.row0 = d0.w;
  ta.M = d1.x;
  ta.n0 = d1.y;
  ta.spl = d1.z;
  ta.ks = d1.w;
  ta.unit0 = d2.x;
  tb.group = d2.y;
  tb.e = d2.z;
  tb.row0 = d2.w;
  tb.M = d3.x;
  tb.n0 = d3.y;
  tb.spl = 1;
  tb.ks = 0;
  tb.unit0 = -1;
  return d0.x;
}

// ----------------------------------------------------------------- bf16 MFMA

// Small-segment kernel (decode-like launches: few rows per expert, so the
// cost is streaming the weights). BM x BN tile, 4 waves in WM x WN. The
// operand rows are copied global -> LDS with global_load_lds (8 rows of 128
// contiguous bytes per instruction) into a ring of NS stages of BK = 64, so
// NS - 1 stages of weights are in flight per workgroup (two workgroups fit a
// CU). Chunk c of row r sits at slot c ^ ((r >> 1) & 7): the 16 lanes served
// together by a 128-bit read (16 consecutive rows, one chunk) hit 16
// distinct 4-bank groups.
template <int BM, int BN>
struct SmallTileShape {
  static constexpr int BK = 64;                           // bf16 elements per K step
  static constexpr int ROWB = BK * 2;                     // bytes per staged row (128)
  static constexpr int STAGE = (BM + BN) * ROWB;
  static constexpr int NS = 3;                            // stages (2 workgroups per CU)
  static constexpr int LDS = NS * STAGE;
};

// One small tile computed by 4 waves (wave = 0..3 inside them) with the
// operand ring at smem. Every LDS hand-off is a workgroup barrier, so all the
// waves of the workgroup must run the same number of K stages (the paired
// tiles of the large-tile kernel share their K). store = false runs the tile
// without writing C (the idle half of an unpaired slot). With part, the
// workgroup computes K slice ks of nks and writes its fp32 partial tile
// ([BM][BN], rows past M and columns past N left unwritten) there instead of C.
template <int BM, int BN, int WM, int WN>
__device__ __forceinline__ void small_tile(const GemmArgs& args, const Tile& t, uint8_t* smem,
                                           int wave, bool store, int ks = 0, int nks = 1,
                                           float* part = nullptr) {
  using Sh = SmallTileShape<BM, BN>;
  constexpr int BK = Sh::BK, ROWB = Sh::ROWB, STAGE = Sh::STAGE, NS = Sh::NS;
  constexpr int WTM = BM / WM, WTN = BN / WN; // wave tile
  constexpr int SM = WTM / 32, SN = WTN / 32; // 32x32 sub-tiles per wave
  constexpr int NI = (BM + BN) / 8 / 4;       // DMA instructions per wave per stage
  static_assert(WM * WN <= 4, "at most 4 computing waves");
  static_assert(SM >= 1 && SN >= 1, "tile shape");
  static_assert((BM + BN) % 32 == 0 && NI >= 1 && NI * (NS - 2) < 64, "whole DMA instructions");
  const Group G = pick_group(args, t.group);
  const int N = G.N, K = G.K;
  const uint16_t* A = static_cast<const uint16_t*>(G.A);
  const uint16_t* B = static_cast<const uint16_t*>(G.B) + (size_t)t.e * N * K + (size_t)t.n0 * K;
  uint16_t* C = static_cast<uint16_t*>(G.C) + (size_t)t.row0 * N + t.n0;
  const int M = t.M;

  const int lane = threadIdx.x & 63;
  // waves WM*WN .. 3 only take part in the copies (narrow tiles for few rows)
  const bool computes = wave < WM * WN;
  const int wm = computes ? wave / WN : 0, wn = computes ? wave % WN : 0;

  // DMA plan: instruction q of this wave fills rows [8g, 8g + 8) of a stage
  // (A rows first, then B rows); lane i takes row 8g + i/8, slot i%8.
  const uint16_t* src[NI];
  int dst[NI];
#pragma unroll
  for (int q = 0; q < NI; ++q) {
    const int g = wave * NI + q;
    const int r = 8 * g + (lane >> 3);
    const int chunk = (lane & 7) ^ ((r >> 1) & 7);
    const uint16_t* row = r < BM ? A + a_row(args, t.group, t.row0 + min(r, M - 1)) * K
                                 : B + (size_t)min(r - BM, N - t.n0 - 1) * K;
    src[q] = row + chunk * 8;
    dst[q] = g * 8 * ROWB;
  }
  const int KT0 = K / BK;
  const int kbase = ks * KT0 / nks;
  const int KT = (ks + 1) * KT0 / nks - kbase;
  auto issue = [&](int kt) {
    uint8_t* base = smem + (kt % NS) * STAGE;
#pragma unroll
    for (int q = 0; q < NI; ++q) lds_dma16(src[q] + (kbase + kt) * BK, base + dst[q]);
  };

  f32x16_t acc[SM][SN];
#pragma unroll
  for (int i = 0; i < SM; ++i)
#pragma unroll
    for (int j = 0; j < SN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // Fragment rows (A: tile rows, B: tile columns) of this lane.
  int fa[SM], fb[SN];
#pragma unroll
  for (int i = 0; i < SM; ++i) fa[i] = (wm * WTM + i * 32 + (lane & 31)) * ROWB;
#pragma unroll
  for (int j = 0; j < SN; ++j) fb[j] = (BM + wn * WTN + j * 32 + (lane & 31)) * ROWB;
  const int sw = (lane >> 1) & 7;  // == (row >> 1) & 7 for every fragment row of this lane
  const int khalf = lane >> 5;

#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < KT) issue(st);
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + NS - 2 < KT) wait_vmcnt<(NS - 2) * NI>();
    else wait_vmcnt<0>();
    lds_barrier();  // stage kt landed for every wave; stage kt-1 is no longer read
    if (kt + NS - 1 < KT) issue(kt + NS - 1);
    const uint8_t* cur = smem + (kt % NS) * STAGE;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (!computes) break;
      const int off = ((ks * 2 + khalf) ^ sw) << 4;
      u32x4_t fra[SM], frb[SN];
#pragma unroll
      for (int i = 0; i < SM; ++i) fra[i] = ld16(cur + fa[i] + off);
#pragma unroll
      for (int j = 0; j < SN; ++j) frb[j] = ld16(cur + fb[j] + off);
#pragma unroll
      for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fra[i]),
                                                              as_bf16x8(frb[j]), acc[i][j], 0, 0, 0);
    }
  }

  // Epilogue. 32x32 D layout: lane holds column lane%32 and rows
  // (v/4)*8 + (lane/32)*4 + v%4 of each sub-tile.
  if (!computes || !store) return;
  const bool gelu = args.gelu != 0;
#pragma unroll
  for (int i = 0; i < SM; ++i)
#pragma unroll
    for (int j = 0; j < SN; ++j) {
      const int col = wn * WTN + j * 32 + (lane & 31);
      if (t.n0 + col >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * WTM + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        if (row < M) {
          if (part != nullptr) {
            part[row * BN + col] = acc[i][j][v];
            continue;
          }
          float y = acc[i][j][v];
          if (gelu) y = gelu_bf16(y);
          C[(size_t)row * N + col] = (uint16_t)f32_to_bf16(y);
        }
      }
    }
}

// blockIdx.y: K slice of gridDim.y (split K writes fp32 partial tiles to
// args.part, [workgroup][slice][BM][BN]; gemm_small_reduce_kernel finishes them).
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(GemmArgs args) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[SmallTileShape<BM, BN>::LDS];
  Tile t;
  if (!find_tile<BM, BN>(args, t)) return;
  const int nks = gridDim.y;
  float* part = nks > 1 ? args.part + ((size_t)blockIdx.x * nks + blockIdx.y) * BM * BN : nullptr;
  small_tile<BM, BN, WM, WN>(args, t, smem, threadIdx.x >> 6, true, blockIdx.y, nks, part);
}

// Sums the nks K slices of each split small tile in slice order, then the
// epilogue of small_tile (erf-GeLU if requested, bf16 rounding, rows past the
// segment end and columns past N masked). Same grid as the GEMM launch.
constexpr int kMaxSmallSplit = 8;

template <int BM, int BN>
__global__ __launch_bounds__(kThreads) void gemm_small_reduce_kernel(GemmArgs args, int nks) {
  Tile t;
  if (!find_tile<BM, BN>(args, t)) return;
  const Group G = pick_group(args, t.group);
  const int N = G.N;
  uint16_t* C = static_cast<uint16_t*>(G.C) + (size_t)t.row0 * N + t.n0;
  const float* P = args.part + (size_t)blockIdx.x * nks * BM * BN;
  const bool gelu = args.gelu != 0;
  for (int q = threadIdx.x; q < t.M * BN; q += kThreads) {
    const int row = q / BN, col = q % BN;
    if (t.n0 + col >= N) continue;
    float v[kMaxSmallSplit];
#pragma unroll
    for (int s = 0; s < kMaxSmallSplit; ++s)  // all loads first, then the sum in slice order
      if (s < nks) v[s] = P[(size_t)s * BM * BN + row * BN + col];
    float y = 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxSmallSplit; ++s)
      if (s < nks) y += v[s];
    if (gelu) y = gelu_bf16(y);
    C[(size_t)row * N + col] = (uint16_t)f32_to_bf16(y);
  }
}

// ----------------------------------------------------------------- bf16 MFMA, few rows

// Row block mt of the routed group: experts in order, each expert's segment
// cut into blocks of BMR rows from its start. One wave finds it (every wave of
// the workgroup runs the same search, so no barrier): each lane sums the blocks
// of 4 consecutive experts (E <= 256), a wave scan orders the lanes, and the
// lane whose range holds mt names the expert. Returns the expert (row0, M:
// the block's first buffer row and row count), or -1 past the last block.
template <int BMR>
__device__ __forceinline__ int find_row_block(const GemmArgs& a, int mt, int& row0, int& M) {
  constexpr int EPL = 4;
  const int lane = threadIdx.x & 63;
  int off[EPL], cnt[EPL], nb[EPL], sum = 0;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane * EPL + j;
    off[j] = 0;
    cnt[j] = 0;
    if (e < a.E) {
      // clamped like find_tile: a segment never leaves the buffer
      off[j] = min(max(a.offsets[e], 0), a.rows);
      cnt[j] = min(max(a.offsets[e + 1], off[j]), a.rows) - off[j];
    }
    nb[j] = (cnt[j] + BMR - 1) / BMR;
    sum += nb[j];
  }
  int incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  const int excl = incl - sum;
  const bool mine = mt >= excl && mt < incl;
  const uint64_t owner = __ballot(mine);
  if (owner == 0) return -1;
  const int src = __ffsll((unsigned long long)owner) - 1;
  int e = 0, r0 = 0, m = 0, base = excl;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    if (mine && mt >= base && mt < base + nb[j]) {
      e = lane * EPL + j;
      r0 = off[j] + (mt - base) * BMR;
      m = min(BMR, cnt[j] - (mt - base) * BMR);
    }
    base += nb[j];
  }
  row0 = __shfl(r0, src);
  M = __shfl(m, src);
  return __shfl(e, src);
}

// Few-row kernel (decode: a few tokens per expert, so a launch is a stream of
// the weights). A workgroup takes a block of up to 16 * R rows of one group
// and 16 * (4 / KQ) columns; each of its 4 waves takes 16 of those columns
// and one of KQ slices of K. Weights go from memory straight to registers (no
// LDS staging: no other wave reads them), one 16-byte load per lane per 16
// columns x 32 k, in chunks of U loads with the next chunk in flight while
// the current one is multiplied. v_mfma_f32_16x16x32_bf16 takes the weights as
// its A operand (16 columns) and the token rows as B (16 rows): lane l loads
// column l % 16 and row l % 16 at k = 8 * (l / 16) of each 32-deep step, the
// same k for both operands. Rows past the block's end read its last row and
// their results are not stored (each output row depends on its own input row
// alone). The KQ partial sums of a column block are added in slice order
// through LDS, then erf-GeLU (up projection) and bf16 rounding; lane l stores
// 4 adjacent columns of row l % 16.
template <int R, int KQ, int U>
__global__ __launch_bounds__(kThreads) void gemm_bf16_rows_kernel(GemmArgs args) {
  constexpr int BMR = 16 * R, NC = 16 * (4 / KQ);
  static_assert(KQ == 1 || KQ == 2 || KQ == 4, "K slices per workgroup");
  __shared__ f32x4_t red[4][R][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = blockIdx.x;
  int group, e, row0, M, n0;
  if (g >= args.routed_tiles) {
    const int gs = g - args.routed_tiles;
    const int ntn = args.shared.N / NC;
    group = 1;
    e = 0;
    row0 = (gs / ntn) * BMR;
    M = min(BMR, args.shared_M - row0);
    n0 = (gs % ntn) * NC;
    if (M <= 0) return;
  } else {
    const int ntn = args.routed.N / NC;
    group = 0;
    e = find_row_block<BMR>(args, g / ntn, row0, M);
    if (e < 0) return;
    n0 = (g % ntn) * NC;
  }
  const Group G = pick_group(args, group);
  const int N = G.N, K = G.K;
  const int cb = wave / KQ, q = wave % KQ;
  const int Ks = K / KQ;
  const int kc = q * Ks + (lane >> 4) * 8;
  const uint16_t* wp =
      static_cast<const uint16_t*>(G.B) + ((size_t)e * N + n0 + cb * 16 + (lane & 15)) * K + kc;
  const uint16_t* xp[R];
#pragma unroll
  for (int rb = 0; rb < R; ++rb)
    xp[rb] = static_cast<const uint16_t*>(G.A) +
             a_row(args, group, row0 + min(rb * 16 + (lane & 15), M - 1)) * K + kc;

  f32x4_t acc[R];
#pragma unroll
  for (int rb = 0; rb < R; ++rb) acc[rb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  u32x4_t wa[U], xa[U][R], wb[U], xb[U][R];
  const int nch = Ks / (32 * U);
#define MOE_ROWS_LOAD(W, X, c)                                   \
  _Pragma("unroll") for (int u = 0; u < U; ++u) {                \
    const int k = ((c) * U + u) * 32;                            \
    W[u] = ld16(wp + k);                                         \
    _Pragma("unroll") for (int rb = 0; rb < R; ++rb) X[u][rb] = ld16(xp[rb] + k); \
  }
#define MOE_ROWS_MMA(W, X)                                                                  \
  _Pragma("unroll") for (int u = 0; u < U; ++u)                                             \
  _Pragma("unroll") for (int rb = 0; rb < R; ++rb) acc[rb] =                                \
      __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(W[u]), as_bf16x8(X[u][rb]), acc[rb], 0, 0, 0);
  MOE_ROWS_LOAD(wa, xa, 0)
  for (int c = 0; c < nch; c += 2) {
    if (c + 1 < nch) { MOE_ROWS_LOAD(wb, xb, c + 1) }
    MOE_ROWS_MMA(wa, xa)
    if (c + 2 < nch) { MOE_ROWS_LOAD(wa, xa, c + 2) }
    if (c + 1 < nch) { MOE_ROWS_MMA(wb, xb) }
  }
#undef MOE_ROWS_LOAD
#undef MOE_ROWS_MMA

  if constexpr (KQ > 1) {
    if (q != 0) {
#pragma unroll
      for (int rb = 0; rb < R; ++rb) red[wave][rb][lane] = acc[rb];
    }
    __syncthreads();
    if (q != 0) return;
#pragma unroll
    for (int sl = 1; sl < KQ; ++sl)
#pragma unroll
      for (int rb = 0; rb < R; ++rb) acc[rb] += red[wave + sl][rb][lane];
  }
  const bool gelu = args.gelu != 0;
  uint16_t* C = static_cast<uint16_t*>(G.C);
#pragma unroll
  for (int rb = 0; rb < R; ++rb) {
    const int r = rb * 16 + (lane & 15);
    if (r >= M) continue;
    float y[4] = {acc[rb][0], acc[rb][1], acc[rb][2], acc[rb][3]};
    if (gelu) {
#pragma unroll
      for (int v = 0; v < 4; ++v) y[v] = gelu_bf16(y[v]);
    }
    const uint2 out = make_uint2(cvt_bf16x2(y[0], y[1]), cvt_bf16x2(y[2], y[3]));
    *reinterpret_cast<uint2*>(C + (size_t)(row0 + r) * N + n0 + cb * 16 + 4 * (lane >> 4)) = out;
  }
}

// ----------------------------------------------------------------- bf16 MFMA, large tiles

// Epilogue of a 256-column big tile computed by NW waves in a 2 x (NW/2)
// grid (wave tile (BM/2) x (BN/(NW/2)) of 32x32 accumulators): one K slice of
// a split tail tile writes its fp32 partial tile; otherwise erf-GeLU (up
// projection), bf16 rounding and coalesced row stores through an LDS tile.
template <int BM, int BN, int NW, bool GELU, int SM, int SN>
__device__ __forceinline__ void big_tile_epilogue(const GemmArgs& args, const Tile& t, uint16_t* C,
                                                  int N, int M, int nvalid,
                                                  f32x16_t (&acc)[SM][SN], uint8_t* smem) {
  constexpr int WN_ = NW / 2;
  constexpr int WTM = BM / 2, WTN = BN / WN_;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN_, wn = wave % WN_;
  if (t.unit0 >= 0) {
    // one K slice of a split tail tile: the fp32 partial tile, row-major,
    // goes to its slot; the reduce launch sums the slices and runs the epilogue
    float* P = args.part + (size_t)(t.unit0 + t.ks) * BM * BN;
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
      for (int j = 0; j < SN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * WTM + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
          const int col = wn * WTN + j * 32 + (lane & 31);
          P[(size_t)row * BN + col] = acc[i][j][v];
        }
    return;
  }

  // Epilogue through LDS. 32x32 D layout: lane holds column lane%32 and rows
  // (v/4)*8 + (lane/32)*4 + v%4. Each lane converts its rows (v, v+1) of its
  // column to a bf16 pair in one instruction; lanes 2m and 2m+1 (adjacent
  // columns) swap those words with DPP, and a byte permute leaves the even
  // lane the pair (row R(v), its column and the next) and the odd lane the
  // same for row R(v) + 1. The pairs go to a [BM x BN] bf16 tile in LDS (the
  // operand stages are free by then), 512-byte rows whose 16-dword groups are
  // XOR-swizzled by row bits 0 and 2: the four rows one write instruction
  // touches (r, r+1, r+4, r+5) land in four different bank quarters. Those
  // two row bits are the lane's parity and lane / 32 for every value, so the
  // swizzled address is a per-lane base plus a constant. Then every wave
  // stores whole rows, 16 bytes per lane (two 512-byte rows per instruction).
  static_assert(BN == 256, "C tile in LDS: 512-byte rows");
  constexpr int CROWB = BN * 2;
  const int odd = lane & 1, hi = lane >> 5;
  const int cg = odd | (hi << 1);  // == (row & 1) | ((row >> 2) & 1) << 1 for this lane's rows
  const int rbase = wm * WTM + hi * 4 + odd;
  int cbase[SN];
#pragma unroll
  for (int j = 0; j < SN; ++j)
    cbase[j] = rbase * CROWB + (((wn * WTN + j * 32) / 32) ^ cg) * 64 + ((lane & 31) >> 1) * 4;
  // even lane: low halves of (own, partner); odd lane: high halves of (partner, own)
  const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
  lds_barrier();  // every wave has read the last stage
#pragma unroll
  for (int i = 0; i < SM; ++i)
#pragma unroll
    for (int j = 0; j < SN; ++j)
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        float y0 = acc[i][j][v], y1 = acc[i][j][v + 1];
        if constexpr (GELU) {
          y0 = gelu_bf16(y0);
          y1 = gelu_bf16(y1);
        }
        const uint32_t own = cvt_bf16x2(y0, y1);  // (row R(v), row R(v) + 1) of this column
        const uint32_t partner = __builtin_amdgcn_mov_dpp(own, 0xB1, 0xF, 0xF, true);
        const uint32_t pair = __builtin_amdgcn_perm(partner, own, sel);
        const int roff = (i * 32 + (v >> 2) * 8 + (v & 3)) * CROWB;
        *reinterpret_cast<uint32_t*>(smem + cbase[j] + roff) = pair;
        // two accumulator pairs at a time: keeps the scheduler from reading
        // every accumulator out to VGPRs ahead of its conversion, while four
        // independent GeLU chains fill the VALU pipeline (one pair at a time:
        // the FFN 0.8-3 % slower, four: no better than two)
        if constexpr (NW == 4) {
          if ((v & 3) == 2) __builtin_amdgcn_sched_barrier(0);
        }
      }
  lds_barrier();
  const int cl = lane & 31;
  const bool cok = cl * 8 < nvalid;  // N % 64 == 0: 8-column chunks are all or nothing
#pragma unroll 4
  for (int it = 0; it < BM / NW / 2; ++it) {
    const int row = wave * (BM / NW) + it * 2 + hi;
    const int rg = (row & 1) | (((row >> 2) & 1) << 1);
    const u32x4_t v = ld16(smem + row * CROWB + (((cl >> 2) ^ rg) << 6) + ((cl & 3) << 4));
    if (cok && row < M) st16(C + (size_t)row * N + cl * 8, v);
  }
}

// Large-tile kernel: BM x BN tile, NW waves in a 2 x (NW/2) grid, each wave a
// (BM/2) x (BN/(NW/2)) block of 32x32x16 MFMAs. Two LDS stages of BK = 64; a
// row of a staged tile is 64 bf16 = 8 chunks of 16 bytes.
// Fragment registers are double buffered across the four 16-deep k slices of
// a stage, and the one barrier per stage sits where every wave already holds
// the old stage's last fragments in registers: after it the old stage is
// refilled (k-step kt+2) and the first fragments of the new stage are read.
template <int BM, int BN, int NW, bool GELU>
__global__ __launch_bounds__(NW * 64, 1) void gemm_bf16_big_kernel(GemmArgs args) {
  constexpr int BK = 64;
  constexpr int ROWB = BK * 2;                  // 128 bytes = 8 chunks of 16
  constexpr int WN_ = NW / 2;
  constexpr int WTM = BM / 2, WTN = BN / WN_;
  constexpr int SM = WTM / 32, SN = WTN / 32;
  constexpr int STAGE = (BM + BN) * ROWB;
  constexpr int ROWS_PER_INST = 64 * 16 / ROWB;   // 8 rows per load instruction
  constexpr int A_INST = BM / ROWS_PER_INST / NW;  // per wave per stage
  constexpr int B_INST = BN / ROWS_PER_INST / NW;
  constexpr int NLD = A_INST + B_INST;
  static_assert(A_INST >= 1 && B_INST >= 1 && SM >= 1 && SN >= 1, "tile shape");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  Tile t, tb;
  const int kind = table_entry(args, blockIdx.x, t, tb);
  if (kind < 0) return;
  if (kind == 1) {
    // two small tiles of short segments, one per half of the waves, each with
    // its own LDS ring (the same K, so both halves meet the same barriers); a
    // slot without a second tile runs the first one twice and stores it once
    static_assert(NW == 8 && 2 * SmallTileShape<kSBM, kSBN>::LDS <= 2 * STAGE, "two small rings");
    const int half = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 8));
    const bool has_b = tb.M > 0;
    small_tile<kSBM, kSBN, 1, 4>(args, half && has_b ? tb : t,
                                 smem + half * SmallTileShape<kSBM, kSBN>::LDS,
                                 (threadIdx.x >> 6) & 3, half == 0 || has_b);
    return;
  }
  const Group G = pick_group(args, t.group);
  const int N = G.N, K = G.K;
  const uint16_t* A = static_cast<const uint16_t*>(G.A);
  const uint16_t* B = static_cast<const uint16_t*>(G.B) + (size_t)t.e * N * K + (size_t)t.n0 * K;
  uint16_t* C = static_cast<uint16_t*>(G.C) + (size_t)t.row0 * N + t.n0;
  const int M = t.M;
  const int nvalid = N - t.n0;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN_, wn = wave % WN_;

  // Slot p of row r holds chunk p ^ ((r >> 1) & 7). A 128-bit LDS read is
  // served 16 lanes at a time; the 16 consecutive rows of one such group then
  // cover all 64 banks exactly once (row parity picks the half, the swizzle
  // the 16-byte column). Lane i of a load instruction fills slot i & 7 of row
  // r0 + (i >> 3), so it loads chunk (i & 7) ^ ((r >> 1) & 7).
  const int lrow = lane >> 3;
  const uint16_t* ga[A_INST];
  const uint16_t* gb[B_INST];
#pragma unroll
  for (int j = 0; j < A_INST; ++j) {
    const int r = (wave * A_INST + j) * ROWS_PER_INST + lrow;
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    ga[j] = A + a_row(args, t.group, t.row0 + min(r, M - 1)) * K + c * 8;
  }
#pragma unroll
  for (int j = 0; j < B_INST; ++j) {
    const int r = (wave * B_INST + j) * ROWS_PER_INST + lrow;
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    gb[j] = B + (size_t)min(r, nvalid - 1) * K + c * 8;
  }
  // K stages of this workgroup: all of them, or one slice of a split tail tile
  const int KT0 = K / BK;
  const int kbase = t.ks * KT0 / t.spl, kend = (t.ks + 1) * KT0 / t.spl;
  auto issue = [&](int kt) {
    uint8_t* base = smem + (kt & 1) * STAGE;
    const int k0 = (kbase + kt) * BK;
#pragma unroll
    for (int j = 0; j < A_INST; ++j)
      lds_dma16(ga[j] + k0, base + (wave * A_INST + j) * ROWS_PER_INST * ROWB);
#pragma unroll
    for (int j = 0; j < B_INST; ++j)
      lds_dma16(gb[j] + k0, base + BM * ROWB + (wave * B_INST + j) * ROWS_PER_INST * ROWB);
  };

  f32x16_t acc[SM][SN];
#pragma unroll
  for (int i = 0; i < SM; ++i)
#pragma unroll
    for (int j = 0; j < SN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  int fa[SM], fb[SN];
#pragma unroll
  for (int i = 0; i < SM; ++i) fa[i] = (wm * WTM + i * 32 + (lane & 31)) * ROWB;
#pragma unroll
  for (int j = 0; j < SN; ++j) fb[j] = (BM + wn * WTN + j * 32 + (lane & 31)) * ROWB;
  const int sw = (lane >> 1) & 7;  // == (row >> 1) & 7 for every fragment row of this lane
  const int khalf = lane >> 5;

  // Row sub-tiles of this wave that hold data (all of them except in a
  // segment's last, partial row tile); empty ones skip reads and MFMAs.
  const int nsub = min(SM, max(0, (M - wm * WTM + 31) / 32));

  u32x4_t ca[SM], cb[SN], na[SM], nb[SN];
  auto main_loop = [&](auto partial_tag) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
    auto load_frags = [&](const uint8_t* st, int ks, u32x4_t (&fa_)[SM], u32x4_t (&fb_)[SN]) {
      const int off = ((ks * 2 + khalf) ^ sw) << 4;
#pragma unroll
      for (int i = 0; i < SM; ++i)
        if (!PARTIAL || i < nsub) fa_[i] = ld16(st + fa[i] + off);
#pragma unroll
      for (int j = 0; j < SN; ++j) fb_[j] = ld16(st + fb[j] + off);
    };
    auto mma = [&](const u32x4_t (&fa_)[SM], const u32x4_t (&fb_)[SN]) {
#pragma unroll
      for (int i = 0; i < SM; ++i)
        if (!PARTIAL || i < nsub)
#pragma unroll
          for (int j = 0; j < SN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fa_[i]), as_bf16x8(fb_[j]),
                                                                acc[i][j], 0, 0, 0);
    };
    const int KT = kend - kbase;
    issue(0);
    if (KT > 1) {
      issue(1);
      wait_vmcnt<NLD>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    load_frags(smem, 0, ca, cb);
    for (int kt = 0; kt < KT; ++kt) {
      const uint8_t* st = smem + (kt & 1) * STAGE;
      load_frags(st, 1, na, nb);
      mma(ca, cb);
      load_frags(st, 2, ca, cb);
      mma(na, nb);
      load_frags(st, 3, na, nb);
      mma(ca, cb);
      if (kt + 1 < KT) {
        // stage kt+1 landed (own loads, then everyone's); stage kt fully in registers
        wait_vmcnt<0>();
        lds_barrier();
        if (kt + 2 < KT) issue(kt + 2);
        load_frags(smem + ((kt + 1) & 1) * STAGE, 0, ca, cb);
      }
      mma(na, nb);
    }
  };
  if (M == BM)
    main_loop(std::integral_constant<bool, false>{});
  else
    main_loop(std::integral_constant<bool, true>{});

  big_tile_epilogue<BM, BN, NW, GELU>(args, t, C, N, M, nvalid, acc, smem);
}

// Large-tile kernel, one wave per SIMD (the default for bf16 launches with
// enough rows): a 256x256 tile, 4 waves, wave w a 128x128 block (rows
// (w/2)*128, columns (w%2)*128) of 4x4 v_mfma_f32_32x32x16_bf16 accumulators
// (all 256 accumulation registers). Against the 8-wave kernel a wave reads
// 8 KB of fragments per 16-deep k slice for 16 MFMAs (6 KB for 8 there): a
// third less LDS read traffic per flop.
//
// With one wave per SIMD nothing else feeds the matrix core, so the stage is
// hand-ordered: every other instruction sits between two MFMAs
// (sched_barrier fences keep the order the source gives).
//   - k slices 1-3 of stage kt each carry the 8 fragment reads of the next
//     slice; after the stage's one barrier, the slice that finishes the stage
//     (k slice 0 of stage kt+1 in registers) carries the 8 reads of the next
//     stage's first slice.
//   - The A rows (tokens) sit in two LDS stage buffers, the B rows (weights)
//     in three. The copies of stage kt+2 go out one every two MFMAs or so: its
//     B rows during the first three slices of stage kt (into the buffer of
//     stage kt-1, freed by the barrier that ended it), its A rows during the
//     last slice, after the barrier that frees their buffer.
//   Measured (FFN alone, one box, alternating runs): issuing all 16 copies of
//   a stage in the last slice left that slice at about half the MFMA rate
//   (per-slice s_memtime stamps: the other three ran at the full rate, the
//   copy waits and the barrier cost 0.4 % and 3 %); spreading them took the
//   dense 8192 x 14336 x 4096 up and down projections from 1052 to 1121
//   TFLOP/s, the fine-grained layer's FFN from 696-712 to 766-777 and the
//   heavy-skew layer's from 906 to 986-1003. A copy every four MFMAs over the
//   whole stage (half of the A rows one slice later) gained nothing more.
//   - Copies take a 32-bit row offset in a VGPR and a scalar base (the host
//     launches this kernel only when every operand buffer is under 4 GiB) and
//     the LDS address in M0, one s_mov and one global_load_lds each.
//   - A segment's last, partial row tile skips the MFMAs of its empty 32-row
//     sub-tiles (a wave-uniform test); its copies and barriers are unchanged.
// Short segments take 256x256 tiles too (the plan has no tile pairs for this
// kernel): copy-bound with their empty sub-tiles' MFMAs skipped, they cost
// about a quarter of the time per column of a pair of 32x128 small tiles run
// one after the other. Split-K slices and the epilogue are the 8-wave kernel's.
template <bool GELU>
__global__ __launch_bounds__(256, 1) void gemm_bf16_w4_kernel(GemmArgs args) {
  constexpr int NW = 4, BM = 256, BN = 256, BK = 64;
  constexpr int ROWB = BK * 2;                     // 128 bytes = 8 chunks of 16
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int SM = WTM / 32, SN = WTN / 32;
  constexpr int RPI = 64 * 16 / ROWB;              // 8 rows per copy instruction
  constexpr int A_INST = BM / RPI / NW;            // copies per wave per stage
  constexpr int B_INST = BN / RPI / NW;
  constexpr int A_STAGE = BM * ROWB, B_STAGE = BN * ROWB;
  constexpr int LDS_BYTES = 2 * A_STAGE + 3 * B_STAGE;
  static_assert(A_INST == 8 && B_INST == 8 && SM == 4 && SN == 4, "tile shape");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS of one workgroup");
  static_assert(BM * BN * 2 <= LDS_BYTES, "the epilogue's C tile fits the stage buffers");
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];

  // every slot holds one big tile or nothing: this kernel's plan has no
  // short-segment pairs (Shape::pairs = 0)
  Tile t, tb;
  if (table_entry(args, blockIdx.x, t, tb) != 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Group G = pick_group(args, t.group);
  const int N = G.N, K = G.K;
  const uint16_t* A = static_cast<const uint16_t*>(G.A);
  const uint16_t* B = static_cast<const uint16_t*>(G.B) + (size_t)t.e * N * K + (size_t)t.n0 * K;
  uint16_t* C = static_cast<uint16_t*>(G.C) + (size_t)t.row0 * N + t.n0;
  const int M = t.M;
  const int nvalid = N - t.n0;
  const int wm = wave >> 1, wn = wave & 1;
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  // Copy plan: copy q of a wave fills 8 rows of a stage buffer, lane i row
  // (wave * 8 + q) * 8 + i / 8, slot i & 7, which holds chunk (i & 7) ^
  // ((r >> 1) & 7) of the row (the XOR swizzle of the 8-wave kernel: the 16
  // lanes a 128-bit LDS read serves together hit all 64 banks once). ov holds
  // the byte offset of the lane's chunk of K stage 0 (A rows, then B rows);
  // rows past the segment end or the column range are clamped.
  const int lrow = lane >> 3;
  uint32_t ov[A_INST + B_INST];
#pragma unroll
  for (int q = 0; q < A_INST; ++q) {
    const int r = (wave * A_INST + q) * RPI + lrow;
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    ov[q] = (uint32_t)((a_row(args, t.group, t.row0 + min(r, M - 1)) * K + c * 8) * 2);
  }
#pragma unroll
  for (int q = 0; q < B_INST; ++q) {
    const int r = (wave * B_INST + q) * RPI + lrow;
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    ov[A_INST + q] = (uint32_t)(((size_t)min(r, nvalid - 1) * K + c * 8) * 2);
  }
  const int KT0 = K / BK;
  const int kbase = t.ks * KT0 / t.spl, kend = (t.ks + 1) * KT0 / t.spl;
  const int KT = kend - kbase;
  const int last = KT - 1;
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) uint8_t*)smem);
  const uint8_t* A8 = reinterpret_cast<const uint8_t*>(A);
  const uint8_t* B8 = reinterpret_cast<const uint8_t*>(B);
  auto a_buf = [&](int kt) { return smem + (kt & 1) * A_STAGE; };
  auto b_buf = [&](int slot) { return smem + 2 * A_STAGE + slot * B_STAGE; };
  // copy q of stage kt (q < 8: A rows into A buffer kt & 1; else B rows into
  // B buffer bslot)
  auto copy = [&](int kt, int bslot, int q) {
    const uint32_t kb = (uint32_t)(kbase + kt) * (BK * 2);
    const uint32_t m0 =
        q < A_INST ? lds0 + (uint32_t)((kt & 1) * A_STAGE + (wv * A_INST + q) * RPI * ROWB)
                   : lds0 + (uint32_t)(2 * A_STAGE + bslot * B_STAGE +
                                       (wv * B_INST + q - A_INST) * RPI * ROWB);
    const uint8_t* base = (q < A_INST ? A8 : B8) + kb;
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(ov[q]), "s"(base), "s"(m0)
                 : "memory");
  };

  f32x16_t acc[SM][SN];
#pragma unroll
  for (int i = 0; i < SM; ++i)
#pragma unroll
    for (int j = 0; j < SN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  int fa[SM], fb[SN];  // LDS byte offsets of this lane's fragment rows in a buffer
#pragma unroll
  for (int i = 0; i < SM; ++i) fa[i] = (wm * WTM + i * 32 + (lane & 31)) * ROWB;
#pragma unroll
  for (int j = 0; j < SN; ++j) fb[j] = (wn * WTN + j * 32 + (lane & 31)) * ROWB;
  const int sw = (lane >> 1) & 7;  // == (row >> 1) & 7 for every fragment row of this lane
  const int khalf = lane >> 5;
  // row sub-tiles of this wave that hold data: all of them except in a
  // segment's last, partial row tile (a wave-uniform count)
  const int nsub = __builtin_amdgcn_readfirstlane(min(SM, max(0, (M - wm * WTM + 31) / 32)));

  u32x4_t ca[SM], cb[SN], na[SM], nb[SN];
  // fragment read r of k slice ks (0..7: b0, a0, b1, b2, b3, a1, a2, a3, the
  // order of first use)
  auto read_r = [&](const uint8_t* sa, const uint8_t* sb, int ks, int r, u32x4_t (&fa_)[SM],
                    u32x4_t (&fb_)[SN]) {
    const int off = ((ks * 2 + khalf) ^ sw) << 4;
    if (r == 0) fb_[0] = ld16(sb + fb[0] + off);
    else if (r == 1) fa_[0] = ld16(sa + fa[0] + off);
    else if (r <= 4) fb_[r - 1] = ld16(sb + fb[r - 1] + off);
    else fa_[r - 4] = ld16(sa + fa[r - 4] + off);
  };
  // NS: the row sub-tiles of this wave that hold data (a compile-time count,
  // so a partial tile's loop has no branch between its MFMAs)
  auto main_loop = [&](auto ns_tag) {
    constexpr int NS = decltype(ns_tag)::value;
    auto mfma_m = [&](auto mc, const u32x4_t (&fa_)[SM], const u32x4_t (&fb_)[SN]) {
      constexpr int m = decltype(mc)::value, i = m >> 2, j = m & 3;
      if constexpr (i < NS)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fa_[i]), as_bf16x8(fb_[j]),
                                                            acc[i][j], 0, 0, 0);
    };
    // One k slice: 16 MFMAs on (fa_, fb_); after each of the first 8 a read
    // of k slice rks of buffers (rsa, rsb) into (ra_, rb_); copies q0 .. q1-1
    // spread evenly over the 16 MFMAs (A rows of stage akt for q < 8, B rows
    // of stage bkt into slot bslot for q >= 8).
    auto slice = [&](const u32x4_t (&fa_)[SM], const u32x4_t (&fb_)[SN], const uint8_t* rsa,
                     const uint8_t* rsb, int rks, u32x4_t (&ra_)[SM], u32x4_t (&rb_)[SN],
                     auto q0c, auto q1c, int akt, int bkt, int bslot) {
      constexpr int q0 = decltype(q0c)::value, nq = decltype(q1c)::value - q0;
      static_for<16>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        mfma_m(mc, fa_, fb_);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (m < 8) {
          read_r(rsa, rsb, rks, m, ra_, rb_);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (nq > 0 && (m * nq) / 16 != ((m + 1) * nq) / 16) {
          constexpr int q = q0 + (m * nq) / 16;
          copy(q < A_INST ? akt : bkt, bslot, q);
          __builtin_amdgcn_sched_barrier(0);
        }
      });
    };
    using I0 = std::integral_constant<int, 0>;
    using I8 = std::integral_constant<int, 8>;
    using I11 = std::integral_constant<int, 11>;
    using I14 = std::integral_constant<int, 14>;
    using I16 = std::integral_constant<int, 16>;
    // prologue: stages 0 and 1 and the B rows of stage 2 in flight, in the
    // order the waits count them; stage 0 landed everywhere
    static_for<A_INST + B_INST>([&](auto q) { copy(0, 0, decltype(q)::value); });
    static_for<A_INST + B_INST>([&](auto q) { copy(min(1, last), 1, decltype(q)::value); });
    static_for<B_INST>([&](auto q) { copy(min(2, last), 2, A_INST + decltype(q)::value); });
    wait_vmcnt<A_INST + 2 * B_INST>();
    lds_barrier();
    static_for<8>([&](auto r) { read_r(a_buf(0), b_buf(0), 0, decltype(r)::value, ca, cb); });
    // One code path for every stage: past the end the copies fetch the last
    // stage again into buffers nobody reads any more and the reads fetch a
    // stale buffer (both in bounds and harmless); the copies are drained
    // before the epilogue reuses the LDS.
    int bs = 0;  // B slot of stage kt (kt mod 3)
    for (int kt = 0; kt < KT; ++kt) {
      const int bs1 = bs == 2 ? 0 : bs + 1;
      const int bsp = bs == 0 ? 2 : bs - 1;  // slot of stage kt-1 = stage kt+2
      const int k2 = min(kt + 2, last);
      const uint8_t* sa = a_buf(kt);
      const uint8_t* sb = b_buf(bs);
      slice(ca, cb, sa, sb, 1, na, nb, I8{}, I11{}, 0, k2, bsp);
      slice(na, nb, sa, sb, 2, ca, cb, I11{}, I14{}, 0, k2, bsp);
      slice(ca, cb, sa, sb, 3, na, nb, I14{}, I16{}, 0, k2, bsp);
      // stage kt+1 landed for this wave (only the B copies of stage kt+2
      // issued above may still be in flight), then for everyone; stage kt
      // fully read, so A buffer kt & 1 is free
      wait_vmcnt<B_INST>();
      lds_barrier();
      slice(na, nb, a_buf(kt + 1), b_buf(bs1), 0, ca, cb, I0{}, I8{}, k2, 0, 0);
      bs = bs1;
    }
    wait_vmcnt<0>();
    // every accumulator leaves each variant in its accumulation registers
    // (the untouched ones too), so the variants meet the epilogue with one
    // register assignment
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
      for (int j = 0; j < SN; ++j) asm volatile("" : "+a"(acc[i][j]));
  };
  // A segment's last, partial row tile skips the MFMAs of its empty 32-row
  // sub-tiles. The count is wave-uniform and picks a loop built for it. One
  // loop with a branch around each MFMA had made these tiles 15-20 % slower
  // than full ones despite the skipped work; computing every sub-tile costs
  // power the full tiles then lack (the Mixtral-shaped FFN gains 2.5 %, the
  // fine-grained one loses 6 %), and choosing the count per stage inside one
  // loop spills (per-tile s_memrealtime stamps, FFN timings).
  switch (nsub) {
    case 4: main_loop(std::integral_constant<int, 4>{}); break;
    case 3: main_loop(std::integral_constant<int, 3>{}); break;
    case 2: main_loop(std::integral_constant<int, 2>{}); break;
    case 1: main_loop(std::integral_constant<int, 1>{}); break;
    default: main_loop(std::integral_constant<int, 0>{}); break;
  }
  big_tile_epilogue<BM, BN, NW, GELU>(args, t, C, N, M, nvalid, acc, smem);
}


// Sums the K slices of each split tail tile (slice order) and runs the
// epilogue of the big kernel: erf-GeLU if requested, bf16 rounding, rows past
// the segment end and columns past N masked. kReduceParts workgroups share a
// tile (BM / kReduceParts rows each), so the partials stream through many CUs.
constexpr int kReduceParts = 8;

template <int BM, int BN>
__global__ __launch_bounds__(kThreads) void gemm_tail_reduce_kernel(GemmArgs args) {
  Tile t, tb;
  if (table_entry(args, args.slots + blockIdx.x / kReduceParts, t, tb) != 0) return;
  const Group G = pick_group(args, t.group);
  const int N = G.N;
  uint16_t* C = static_cast<uint16_t*>(G.C) + (size_t)t.row0 * N + t.n0;
  const int nvalid = N - t.n0;
  const bool gelu = args.gelu != 0;
  const float* P = args.part + (size_t)t.unit0 * BM * BN;
  constexpr int RR = BM / kReduceParts;  // rows of this workgroup
  const int r0 = (blockIdx.x % kReduceParts) * RR;
  // 4 columns per thread (N % 64 == 0: a group of 4 is all in or all out);
  // every slice load is issued, from a slice index clamped into [0, spl), before
  // the sum in slice order (guarded loads would each wait in a branch)
  const int spl = t.spl;
  for (int q = threadIdx.x; q < RR * BN / 4; q += kThreads) {
    const int row = r0 + q / (BN / 4), col = (q % (BN / 4)) * 4;
    if (row >= t.M || col >= nvalid) continue;
    f32x4_t v[kMaxSplit];
#pragma unroll
    for (int ks = 0; ks < kMaxSplit; ++ks)
      v[ks] = *reinterpret_cast<const f32x4_t*>(P + (size_t)min(ks, spl - 1) * BM * BN +
                                                (size_t)row * BN + col);
    f32x4_t y = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < kMaxSplit; ++ks)
      if (ks < spl) y += v[ks];
    if (gelu) {
#pragma unroll
      for (int c = 0; c < 4; ++c) y[c] = gelu_bf16(y[c]);
    }
    *reinterpret_cast<uint2*>(C + (size_t)row * N + col) =
        make_uint2(cvt_bf16x2(y[0], y[1]), cvt_bf16x2(y[2], y[3]));
  }
}

// ----------------------------------------------------------------- fp32 VALU

__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmArgs args) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  Tile t;
  if (!find_tile<BM, BN>(args, t)) return;
  const Group G = pick_group(args, t.group);
  const int N = G.N, K = G.K;
  const float* A = static_cast<const float*>(G.A);
  const float* B = static_cast<const float*>(G.B) + (size_t)t.e * N * K + (size_t)t.n0 * K;
  float* C = static_cast<float*>(G.C) + (size_t)t.row0 * N + t.n0;
  const int M = t.M;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int lr = tid >> 2, lk = (tid & 3) * 4;  // loader: row, first k of a float4
  const float* ga = A + a_row(args, t.group, t.row0 + min(lr, M - 1)) * K + lk;
  const float* gb = B + (size_t)min(lr, N - t.n0 - 1) * K + lk;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
    const float4 va = *reinterpret_cast<const float4*>(ga + k0);
    const float4 vb = *reinterpret_cast<const float4*>(gb + k0);
    As[lk + 0][lr] = va.x;
    As[lk + 1][lr] = va.y;
    As[lk + 2][lr] = va.z;
    As[lk + 3][lr] = va.w;
    Bs[lk + 0][lr] = vb.x;
    Bs[lk + 1][lr] = vb.y;
    Bs[lk + 2][lr] = vb.z;
    Bs[lk + 3][lr] = vb.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = ty * 4 + i;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = tx * 4 + j;
      if (t.n0 + col >= N) continue;
      float y = acc[i][j];
      if (args.gelu) y = gelu_erf(y);
      C[(size_t)row * N + col] = y;
    }
  }
}

// ----------------------------------------------------------------- host side

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

template <int BM, int BN>
void grid_of(GemmArgs& a, int rows, int E, dim3& grid) {
  // sum_e ceil(c_e / BM) <= rows / BM + #{e : c_e > 0} <= rows / BM + min(E, rows)
  const int mt_max = rows / BM + min(E, rows);
  a.routed_tiles = mt_max * ((a.routed.N + BN - 1) / BN);
  const int shared_tiles =
      a.shared_M > 0 ? ((a.shared_M + BM - 1) / BM) * ((a.shared.N + BN - 1) / BN) : 0;
  grid = dim3(a.routed_tiles + shared_tiles);
}

// K slices of a small-tile launch. With fewer tiles than CUs (every
// workgroup would walk all of K alone on a CU of its own) K is split so that
// about 1024 workgroups stream the weights, each slice at least 8 stages of
// the routed K; gemm_small_reduce_kernel sums the slices. Measured on the
// graph-replayed decode layer (H = 4096, E = 128, k = 8, F = 1536 + shared),
// which the few-row kernel now runs: T = 1 FFN 55.1 -> 48.7 us (216
// up-projection tiles, 4 slices); at T = 2 (408 tiles) a 2-way split cost
// 3 us more than it saved, hence the limit.
constexpr int kSmallBM = 32, kSmallBN = 64;

int small_splits(const GemmArgs& a, int rows, int E) {
  GemmArgs b = a;
  dim3 grid;
  grid_of<kSmallBM, kSmallBN>(b, rows, E, grid);
  if (grid.x >= (unsigned)(kXcds * kSlots)) return 1;
  const int by_tiles = (int)(1024 / std::max(1u, grid.x));
  const int by_k = a.routed.K / 64 / 8;
  return std::max(1, std::min(std::min(by_tiles, by_k), kMaxSmallSplit));
}

// Records ev on s when given (the caller's timing of one GEMM launch).
hipError_t mark(hipEvent_t ev, hipStream_t s) { return ev ? hipEventRecord(ev, s) : hipSuccess; }

template <int BM, int BN, int WM, int WN>
hipError_t run_bf16(GemmArgs a, int rows, int E, int nks, hipStream_t s, hipEvent_t after) {
  dim3 grid;
  grid_of<BM, BN>(a, rows, E, grid);
  const unsigned nt = grid.x;
  grid.y = nks;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN>), grid, dim3(kThreads), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err == hipSuccess) err = mark(after, s);
  if (err != hipSuccess || nks <= 1) return err;
  hipLaunchKernelGGL((gemm_small_reduce_kernel<BM, BN>), dim3(nt), dim3(kThreads), 0, s, a, nks);
  return hipGetLastError();
}

// Few-row kernel. Workgroups of a launch with 16 * R-row blocks and KQ K
// slices per workgroup (16 * 4 / KQ columns each). kRowsU: loads per chunk of
// a wave's weight stream (two chunks in flight). Measured on the
// graph-replayed decode layer (H = 4096, E = 128, k = 8, F = 1536 + shared),
// FFN at T = 16: 8 loads 401 us, 4 loads 401 us, 2 loads 388 us, 1 load 396 us
// (fewer registers per wave, more waves per SIMD).
constexpr int kRowsU = 2;

template <int R>
int rows_grid(const GemmArgs& a, int rows, int E, int kq) {
  constexpr int BMR = 16 * R;
  const int nc = 16 * (4 / kq);
  // sum_e ceil(c_e / BMR) <= rows / BMR + #{e : c_e > 0}
  const int mt_max = rows / BMR + std::min(E, rows);
  const int shared = a.shared_M > 0 ? ((a.shared_M + BMR - 1) / BMR) * (a.shared.N / nc) : 0;
  return mt_max * (a.routed.N / nc) + shared;
}

// K slices per workgroup: the most of 4, 2, 1 that leave each wave's slice
// whole chunks of kRowsU loads in both groups (0: none fits). More slices
// mean more, shorter weight streams in flight: measured on the graph-replayed
// decode layer (H = 4096, E = 128, k = 8, F = 1536 + shared) at T = 16, FFN
// 396 us with 4 slices against 427 us with the fewest slices that still give
// 1024 workgroups (1 slice, 64-column blocks: each token row read by 4x fewer
// workgroups), both with 8-load chunks.
template <int R>
int rows_kq(const GemmArgs& a, int rows, int E) {
  (void)rows;
  (void)E;
  for (int kq : {4, 2, 1}) {
    const int step = 32 * kRowsU * kq;
    if (a.routed.K % step == 0 && (a.shared_M == 0 || a.shared.K % step == 0)) return kq;
  }
  return 0;
}

// 16-row blocks per workgroup of the few-row kernel for a launch, or 0 for
// the 32 x 64 tile kernel. The few-row kernel reads each token row once per
// 16 columns (the tile kernel: once per 64, through LDS) and every row block
// re-reads its expert's weights, so it pays at up to about two rows per
// expert on average. Measured (decode layer above, graph replay from cold
// caches, few-row kernel against tile kernel): T = 1 77 against 83 us,
// T = 16 415 against 440, T = 32 561 against 573, T = 64 639 against 616,
// T = 128 742 against 629.
int rows_blocks(const GemmArgs& a, int rows, int E) {
  if (rows_kq<1>(a, rows, E) == 0 || a.routed.N % 64 != 0 ||
      (a.shared_M > 0 && a.shared.N % 64 != 0))
    return 0;
  return rows <= 2 * E ? 1 : 0;
}

template <int R, int KQ>
hipError_t run_rows(GemmArgs a, int rows, int E, hipStream_t s, hipEvent_t after) {
  constexpr int BMR = 16 * R, NC = 16 * (4 / KQ);
  a.routed_tiles = (rows / BMR + std::min(E, rows)) * (a.routed.N / NC);
  const int grid = rows_grid<R>(a, rows, E, KQ);
  if (grid > 0)
    hipLaunchKernelGGL((gemm_bf16_rows_kernel<R, KQ, kRowsU>), dim3(grid), dim3(kThreads), 0, s, a);
  const hipError_t err = hipGetLastError();
  return err == hipSuccess ? mark(after, s) : err;
}

template <int R>
hipError_t run_rows_r(const GemmArgs& a, int rows, int E, hipStream_t s, hipEvent_t after) {
  switch (rows_kq<R>(a, rows, E)) {
    case 4: return run_rows<R, 4>(a, rows, E, s, after);
    case 2: return run_rows<R, 2>(a, rows, E, s, after);
    default: return run_rows<R, 1>(a, rows, E, s, after);
  }
}

// One GEMM launch (and its split-K reduce, if any). before / after: events
// recorded right before and right after the GEMM kernel itself, or null.
hipError_t run_gemm(const GemmArgs& a, int rows, int E, bool bf16, bool small_segments,
                    hipStream_t s, hipEvent_t before = nullptr, hipEvent_t after = nullptr) {
  hipError_t err = mark(before, s);
  if (err != hipSuccess) return err;
  if (!bf16) {
    GemmArgs b = a;
    dim3 grid;
    grid_of<64, 64>(b, rows, E, grid);
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(kThreads), 0, s, b);
    err = hipGetLastError();
    return err == hipSuccess ? mark(after, s) : err;
  }
  if (small_segments) {
    if (rows_blocks(a, rows, E) == 1) return run_rows_r<1>(a, rows, E, s, after);
    // 32x64 tiles: 36 KiB rings, so more workgroups per CU keep weight copies
    // in flight than with 32x128 tiles (measured, graph-replayed decode layer,
    // H = 4096, E = 128, k = 8: FFN at T = 128 640 -> 603 us, T = 16 426 ->
    // 412 us, T = 1 unchanged; a four- or five-stage ring gains nothing more)
    const int nks = a.part != nullptr ? small_splits(a, rows, E) : 1;
    return run_bf16<kSmallBM, kSmallBN, 1, 2>(a, rows, E, nks, s, after);
  }
  // big tiles: the table was written by big_plan_kernel. The 4-wave kernel
  // addresses its operand rows with 32-bit offsets; a launch with an operand
  // buffer of 4 GiB or more takes the 8-wave kernel.
  if (a.wide) {
    if (a.gelu)
      hipLaunchKernelGGL((gemm_bf16_big_kernel<256, 256, kBigWaves, true>), dim3(a.slots),
                         dim3(kBigWaves * 64), 0, s, a);
    else
      hipLaunchKernelGGL((gemm_bf16_big_kernel<256, 256, kBigWaves, false>), dim3(a.slots),
                         dim3(kBigWaves * 64), 0, s, a);
  } else if (a.gelu) {
    hipLaunchKernelGGL((gemm_bf16_w4_kernel<true>), dim3(a.slots), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((gemm_bf16_w4_kernel<false>), dim3(a.slots), dim3(256), 0, s, a);
  }
  err = hipGetLastError();
  if (err == hipSuccess) err = mark(after, s);
  if (err != hipSuccess || a.part == nullptr) return err;
  hipLaunchKernelGGL((gemm_tail_reduce_kernel<256, 256>), dim3(kReduceSlots * kReduceParts),
                     dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// The big-tile path (bf16, enough rows per expert) also needs the split-K
// partial tiles and the tile tables.
bool big_tiles(int rows, int E, bool bf16) { return bf16 && (long long)rows >= 64LL * E; }

// Workspace layout: h [rows, F] | hs [T, Fs] | big tiles only: split-K
// partials [kPartTiles, 256, 256] fp32 | tile tables of the up and down launches.
struct FfnLayout {
  GemmArgs up, down;
  size_t h, hs, part, table, bytes;  // byte offsets, total
  bool big, small_segments;
};

// Arguments of both launches and the workspace layout; the same function
// sizes the workspace and launches, so the two always agree.
FfnLayout ffn_layout(const void* xs, const int32_t* gather, int gk, const int32_t* offsets,
                     int rows, int E, int H, int F, const void* w1, const void* w2, const void* x,
                     const void* ws1, const void* ws2, int T, int Fs, bool bf16, void* ys,
                     void* ysh, void* ws) {
  FfnLayout Lo{};
  const size_t es = bf16 ? 2 : 4;
  Lo.big = big_tiles(rows, E, bf16);
  // Few rows per expert on average: decode-like, weight-streaming bound.
  Lo.small_segments = !Lo.big && bf16;
  Lo.h = 0;
  Lo.hs = Lo.h + align256((size_t)rows * F * es);
  Lo.part = Lo.hs + align256((size_t)T * Fs * es);
  Lo.table = Lo.part + (Lo.big ? kPartTiles * 256 * 256 * sizeof(float) : 0);
  uint8_t* base = static_cast<uint8_t*>(ws);
  auto at = [&](size_t off) { return base ? static_cast<void*>(base + off) : nullptr; };
  const bool shared = Fs > 0;

  GemmArgs& up = Lo.up;
  up.routed = Group{xs, w1, at(Lo.h), F, H};
  up.shared = Group{x, ws1, at(Lo.hs), Fs, H};
  up.offsets = offsets;
  up.E = E;
  up.rows = rows;
  up.shared_M = shared ? T : 0;
  up.gelu = 1;
  up.gather = gather;  // routed A = x read through perm (xs is then x)
  up.gk = gk;
  up.gT = T;

  GemmArgs& down = Lo.down;
  down.routed = Group{at(Lo.h), w2, ys, H, F};
  down.shared = Group{at(Lo.hs), ws2, ysh, H, Fs};
  down.offsets = offsets;
  down.E = E;
  down.rows = rows;
  down.shared_M = shared ? T : 0;
  down.gelu = 0;

  size_t table_bytes = 0;
  if (Lo.small_segments) {
    // split-K partial tiles of launches with few small tiles (part stays null
    // for a launch that does not split)
    size_t need = 0;
    for (GemmArgs* a : {&up, &down}) {
      const int nks = small_splits(*a, rows, E);
      if (nks <= 1) continue;
      dim3 grid;
      grid_of<kSmallBM, kSmallBN>(*a, rows, E, grid);
      need = std::max(need, (size_t)grid.x * nks * kSmallBM * kSmallBN * sizeof(float));
    }
    for (GemmArgs* a : {&up, &down})
      a->part = small_splits(*a, rows, E) > 1 ? static_cast<float*>(at(Lo.part)) : nullptr;
    Lo.table = Lo.part + align256(need);
  }
  if (Lo.big) {
    // 32-bit row offsets of the 4-wave kernel: every A buffer under 4 GiB
    const size_t es2 = es;
    const size_t a_up = (size_t)(gather ? T : rows) * H * es2, a_down = (size_t)rows * F * es2;
    const size_t s_up = (size_t)T * H * es2, s_down = (size_t)T * Fs * es2;
    const size_t lim = size_t(1) << 32;
    up.wide = (a_up >= lim || (shared && s_up >= lim)) ? 1 : 0;
    down.wide = (a_down >= lim || (shared && s_down >= lim)) ? 1 : 0;
    int4* tab = static_cast<int4*>(at(Lo.table));
    for (GemmArgs* a : {&up, &down}) {
      // split K only where every group's K is long (plan::split_ok), and the
      // launch's workgroups from the same shape the planner sees
      plan::Shape sh{E, rows, a->shared_M, a->routed.N, a->routed.K, a->shared.N, a->shared.K, 0, 0,
                     a->wide};
      sh.split = plan::split_ok(sh) ? 1 : 0;
      a->part = sh.split ? static_cast<float*>(at(Lo.part)) : nullptr;
      a->slots = plan::launch_slots<256, 256>(sh);
      a->table = tab ? tab + table_bytes / sizeof(int4) : nullptr;
      table_bytes += (size_t)(a->slots + kReduceSlots) * kTableInt4 * sizeof(int4);
    }
  }
  Lo.bytes = Lo.table + align256(table_bytes);
  return Lo;
}

}  // namespace

size_t ffn_ws_bytes(int rows, int T, int E, int H, int F, int Fs, bool bf16) {
  return ffn_layout(nullptr, nullptr, 0, nullptr, rows, E, H, F, nullptr, nullptr, nullptr,
                    nullptr, nullptr, T, Fs, bf16, nullptr, nullptr, nullptr)
      .bytes;
}

hipError_t launch_expert_ffn(const void* xs, const int32_t* gather, int gk,
                             const int32_t* offsets, int rows, int E, int H, int F, const void* w1,
                             const void* w2, const void* x, const void* ws1, const void* ws2,
                             int T, int Fs, bool bf16, void* ys, void* ysh, void* ws,
                             hipStream_t s, void* const* events) {
  hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
  if (events)
    for (int i = 0; i < 4; ++i) ev[i] = static_cast<hipEvent_t>(events[i]);
  const FfnLayout Lo = ffn_layout(xs, gather, gk, offsets, rows, E, H, F, w1, w2, x, ws1, ws2, T,
                                  Fs, bf16, ys, ysh, ws);
  hipError_t err;
  if (Lo.big) {
    const int n = std::max(Lo.up.slots, Lo.down.slots) + kReduceSlots;
    hipLaunchKernelGGL((big_plan_kernel<256, 256, kBlockCols>), dim3((n + kThreads - 1) / kThreads, 2),
                       dim3(kThreads), 0, s, Lo.up, Lo.down);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  err = run_gemm(Lo.up, rows, E, bf16, Lo.small_segments, s, ev[0], ev[1]);
  if (err != hipSuccess) return err;
  return run_gemm(Lo.down, rows, E, bf16, Lo.small_segments, s, ev[2], ev[3]);
}

}  // namespace moe

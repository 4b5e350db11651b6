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
// Two bf16 kernels, both v_mfma_f32_32x32x16_bf16 with fp32 accumulation and
// operands copied global -> LDS by global_load_lds (8 rows of 128 contiguous
// bytes per instruction), 16-byte chunks XOR-swizzled by row so fragment
// reads are bank-conflict free; rows past the segment end are clamped on load
// and masked on store:
//   gemm_bf16_big_kernel   256x256 tiles, 8 waves, two LDS stages, blocked
//                          XCD-aware tile order, split K in the last round of
//                          long-K launches (gemm_tail_reduce_kernel sums it);
//                          segments of at most 32 rows as pairs of 32x128
//                          tiles, one per half of the waves;
//   gemm_bf16_kernel       32x64 tiles for launches with few rows per expert
//                          (decode): weight streaming through a 3-stage ring,
//                          split over K when there are fewer tiles than CUs
//                          (gemm_small_reduce_kernel sums the slices).
// fp32 path (small fp32 layers): 64x64 tiles of plain FMA.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"


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

struct Tile {
  int group;  // 0 routed, 1 shared
  int e;      // expert (routed)
  int row0;   // first row of the tile in A / C
  int M;      // valid rows in this tile (<= BM)
  int n0;     // first column
  int spl;    // K slices of this tile (1: the whole K in one workgroup)
  int ks;     // this workgroup's slice
  int unit0;  // partial-tile index of slice 0 (split tiles), else -1
};

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

// Blocked, XCD-aware tile order (large tiles). Groups are the E experts and
// then the shared expert. A group with c rows has ceil(c/BM) row tiles; if BM
// does not divide c the last one is partial (it skips the 32-row sub-tiles
// past the segment end).
//
// Inside a group tiles are visited in n-blocks of GN column tiles, row tile by
// row tile inside an n-block (consecutive tiles share A rows and cycle
// through GN weight panels). A partial row tile sits in the n-blocks with the
// full ones, so it reads each weight panel while the others of its n-block
// do, not again after every panel has left the caches. Workgroups are handed
// to the 8 XCDs round robin (workgroup g runs on XCD g % 8); XCD x takes the
// contiguous run [x*C, (x+1)*C) of this order (C = ceil(tiles/8)), so the ~32
// tiles an XCD runs at once form a compact block whose operand panels its L2
// shares.
//
// Split K in the last round: an XCD runs S = C tiles, kSlots at a time.
// When the last round holds tail = S mod kSlots tiles and that is at most half
// a round, each of those tiles is cut into spl K slices (one workgroup each,
// spl = kSlots / tail, at most kMaxSplit, and every slice keeps at least
// kMinSliceStages K stages). A slice writes its fp32 partial tile to a.part;
// a second launch (mode 1) sums the spl partials of each tail tile in slice
// order and runs the epilogue. The partition depends only on the counts, so
// results repeat bit for bit. Only long K qualifies (every group's K at least
// kSplitMinK): a short tail tile does not repay the partial round trip and
// the extra launch (measured on the fine-grained and heavy-skew layers).
constexpr int kXcds = 8;
constexpr int kSlots = 32;    // CUs per XCD: workgroups one round of an XCD runs
constexpr int kMaxSplit = 8;
constexpr int kMinSliceStages = 32;  // a slice writes a 256 KB partial: keep it worth it
constexpr int kSplitMinK = 8192;
constexpr int kBigWaves = 8;
// GN of the tile order: column tiles per n-block. Measured against 8 (FFN,
// same box, two alternating runs): Mixtral-shaped 2162-2166 -> 2133 us,
// fine-grained 1227-1231 -> 1216 us, heavy-skew unchanged; 16 was 3% slower
// on the Mixtral-shaped layer, 2 1-2% slower on the heavy-skew one.
constexpr int kBlockCols = 4;
constexpr size_t kPartTiles = (size_t)kXcds * kSlots;  // split units at most

// Small segments inside a big-tile launch. A routed segment of at most 32
// rows would fill one of the 8 sub-tile rows of a 256x256 tile while the tile
// streams the whole weight panel and copies 256 (clamped) A rows. Such
// segments run as 32 x 128 tiles (kSBM x kSBN) instead, two per workgroup (one
// per half of the 8 waves, each with its own LDS ring), and their slots are
// spread evenly through each XCD's sequence among the big tiles. Measured on
// the fine-grained and heavy-skew layers: 1-2% off the FFN; a 128-row limit
// (up to 4 strips re-reading the same weights) was 3% slower than none. Not in
// split-K launches, and not for the shared group (the two tiles of a
// workgroup must have the same K: they meet the same barriers). If the
// launch's slots cannot hold the pairs, every segment takes big tiles.
constexpr int kSmallRows = 33;
constexpr int kSBM = 32, kSBN = 128;

// Tables of the big-tile schedule (per workgroup, in LDS).
struct SchedLds {
  int pf[257];               // inclusive scan of the big tiles by group (small mode)
  int pa[257];               // the same when every segment takes big tiles
  int ps[257];               // inclusive scan of the small tiles by group
  int goff[257], gcnt[257];  // first row and rows of each group
};

struct BigSched {
  const int* pf;     // big-tile scan in use
  int F, CF;         // big tiles in all; per XCD
  int P, CP;         // small-tile pairs in all; per XCD
  int R, tail, spl;  // whole rounds per XCD, tiles of the last round, K slices of those
};

// Computes the schedule of a big-tile launch: the same for every workgroup,
// and for every tile a workgroup runs.
template <int BM, int BN>
__device__ BigSched big_schedule(const GemmArgs& a, SchedLds& L) {
  // Only the first 256 threads take part (the workgroup may be larger);
  // every thread still meets every barrier.
  const int tid = threadIdx.x;
  const bool act = tid < 256;
  const int ng = a.E + (a.shared_M > 0 ? 1 : 0);
  const int ntr = (a.routed.N + BN - 1) / BN;
  const int nts = (a.shared.N + BN - 1) / BN;
  const int nsr = (a.routed.N + kSBN - 1) / kSBN;
  const bool small_ok = a.part == nullptr;
  // thread e: expert e; thread E: the shared group; thread 255 also carries
  // the shared group as group 256 when E == 256
  auto rows_of = [&](int grp, int& off, int& cnt) {
    if (grp < a.E) {
      off = min(max(a.offsets[grp], 0), a.rows);
      cnt = min(max(a.offsets[grp + 1], off), a.rows) - off;
    } else {
      off = 0;
      cnt = a.shared_M;
    }
  };
  int off = 0, cnt = 0, all = 0, big = 0, sml = 0;
  if (act && tid < ng) {
    rows_of(tid, off, cnt);
    all = ((cnt + BM - 1) / BM) * (tid < a.E ? ntr : nts);
    const bool small = small_ok && tid < a.E && cnt > 0 && cnt < kSmallRows;
    big = small ? 0 : all;
    sml = small ? ((cnt + kSBM - 1) / kSBM) * nsr : 0;
  }
  const int xtiles = (tid == 255 && ng == 257) ? ((a.shared_M + BM - 1) / BM) * nts : 0;
  if (act) {
    L.goff[tid] = off;
    L.gcnt[tid] = cnt;
    L.pa[tid] = all;
    L.pf[tid] = big;
    L.ps[tid] = sml;
  }
  if (tid == 255) {
    L.goff[256] = 0;
    L.gcnt[256] = ng == 257 ? a.shared_M : 0;
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
    L.pa[256] = L.pa[255] + xtiles;
    L.pf[256] = L.pf[255] + xtiles;
    L.ps[256] = L.ps[255];
  }
  __syncthreads();
  const int last = ng <= 256 ? ng - 1 : 256;
  BigSched S;
  const int Fs = L.pf[last], Ps = (L.ps[last] + 1) / 2;
  const int CFs = (Fs + kXcds - 1) / kXcds, CPs = (Ps + kXcds - 1) / kXcds;
  if (Ps > 0 && kXcds * (CFs + CPs) <= a.slots && CFs + CPs < (1 << 15)) {
    S.pf = L.pf;
    S.F = Fs;
    S.P = Ps;
  } else {
    S.pf = L.pa;
    S.F = L.pa[last];
    S.P = 0;
  }
  S.CF = (S.F + kXcds - 1) / kXcds;
  S.CP = (S.P + kXcds - 1) / kXcds;
  S.R = S.CF / kSlots;
  S.tail = S.CF - S.R * kSlots;
  S.spl = 1;
  if (a.part != nullptr && S.tail > 0 && 2 * S.tail <= kSlots) {  // a.part: K long enough
    int ktmin = a.routed.K / 64;
    if (a.shared_M > 0) ktmin = min(ktmin, a.shared.K / 64);
    S.spl = max(1, min(min(kSlots / S.tail, kMaxSplit), ktmin / kMinSliceStages));
  }
  return S;
}

// The first entry of an inclusive scan over groups [0, ng) above q.
__device__ __forceinline__ int scan_find(const int* scan, int ng, int q) {
  int lo = 0, hi = ng - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (scan[mid] > q) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// Small tile u of the launch (u < number of small tiles).
__device__ __forceinline__ void small_tile_of(const GemmArgs& a, const SchedLds& L, int u,
                                              Tile& t) {
  const int grp = scan_find(L.ps, a.E, u);
  const int li = u - (grp ? L.ps[grp - 1] : 0);
  const int c = L.gcnt[grp];
  const int nrs = (c + kSBM - 1) / kSBM;  // row strips of the segment
  const int r = li % nrs;
  t.group = 0;
  t.e = grp;
  t.row0 = L.goff[grp] + r * kSBM;
  t.M = min(kSBM, c - r * kSBM);
  t.n0 = (li / nrs) * kSBN;
  t.spl = 1;
  t.ks = 0;
  t.unit0 = -1;
}

// Slot `slot` on XCD x, resolved by one thread from the schedule tables.
// mode 0: the launch's work, kind 0 = one big tile (or K slice of a split
// tail tile) in ta, kind 1 = a pair of small tiles (ta, and tb unless
// tb.M == 0); mode 1: the split tail tile number `slot` to reduce (kind 0).
// Returns -1 if the slot holds nothing.
// An XCD runs CF big-tile slots and CP pair slots; pair slots sit at the
// positions s where floor((s + 1) * CP / n) steps (n = CF + CP), evenly
// spread.
template <int BM, int BN, int GN>
__device__ int resolve_slot(const GemmArgs& a, const BigSched& S, const SchedLds& L, int x,
                            int slot, int mode, Tile& ta, Tile& tb) {
  const int ng = a.E + (a.shared_M > 0 ? 1 : 0);
  const int ntr = (a.routed.N + BN - 1) / BN;
  const int nts = (a.shared.N + BN - 1) / BN;
  const int F = S.F, CF = S.CF, R = S.R, tail = S.tail, spl = S.spl;
  int ks = 0, unit0 = -1;
  if (mode == 0) {
    if (S.CP > 0) {  // pairs (never with split K, whose slices sit past CF)
      const int n = CF + S.CP;
      if (slot >= n) return -1;
      // slot < n < 2^15 and CP < 2^15 (pairs only then): the products fit 32 bits
      const int pb = (int)((unsigned)(slot * S.CP) / (unsigned)n);
      if ((int)((unsigned)((slot + 1) * S.CP) / (unsigned)n) > pb) {  // a pair slot
        const int p = pb * kXcds + x;
        if (p >= S.P) return -1;
        const int nsm = L.ps[a.E - 1];
        small_tile_of(a, L, 2 * p, ta);
        if (2 * p + 1 < nsm) small_tile_of(a, L, 2 * p + 1, tb);
        else tb.M = 0;
        return 1;
      }
      slot -= pb;  // big-tile slots before this one
    }
    if (spl > 1 && slot >= R * kSlots) {
      const int u = slot - R * kSlots;
      if (u >= tail * spl) return -1;
      const int tt = u / spl;
      ks = u - tt * spl;
      slot = R * kSlots + tt;
      unit0 = x * kSlots + tt * spl;
    }
  } else {
    if (spl <= 1 || slot >= tail) return -1;
    unit0 = x * kSlots + slot * spl;
    slot = R * kSlots + slot;
  }
  if (slot >= CF) return -1;
  const int q = x * CF + slot;
  if (q >= F) return -1;
  const int grp = scan_find(S.pf, ng, q);
  const int excl = grp ? S.pf[grp - 1] : 0;
  const int o = L.goff[grp], c = L.gcnt[grp];
  const int mt_g = (c + BM - 1) / BM;  // row tiles of the group, the last one maybe partial
  const int nt_g = grp < a.E ? ntr : nts;
  const int local = q - excl;
  const int blk = local / (mt_g * GN);
  const int w = min(GN, nt_g - blk * GN);
  const int li = local - blk * mt_g * GN;
  ta.row0 = o + (li / w) * BM;
  ta.M = min(BM, c - (li / w) * BM);
  ta.n0 = (blk * GN + li % w) * BN;
  ta.group = grp < a.E ? 0 : 1;
  ta.e = grp < a.E ? grp : 0;
  ta.spl = unit0 >= 0 ? spl : 1;
  ta.ks = ks;
  ta.unit0 = unit0;
  return 0;
}

// Split tail tiles a reduce launch can hold: half a round of every XCD.
constexpr int kReduceSlots = kXcds * kSlots / 2;
constexpr int kTableInt4 = 4;  // int4 per table entry

// Writes the tile table of one big-tile launch, four int4 per workgroup slot:
// {kind, group a, expert a, row0 a}, {M a, n0 a, spl, ks},
// {unit0, group b, expert b, row0 b}, {M b, n0 b, 0, 0} (kind -1: nothing,
// 0: a big tile in a, 1: small tiles a and b, b absent if M b = 0); slots
// [0, a.slots) for the GEMM launch (workgroup g: slot g / 8 on XCD g % 8), then
// kReduceSlots for its split-K reduce. Every workgroup computes the same
// schedule (group scans, from offsets), then each thread resolves one slot:
// the GEMM workgroups read one entry instead of each redoing the schedule.
template <int BM, int BN, int GN>
__device__ void plan_launch(const GemmArgs& a, int4* table, SchedLds& L) {
  const BigSched S = big_schedule<BM, BN>(a, L);
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= a.slots + kReduceSlots) return;
  const int mode = i < a.slots ? 0 : 1;
  const int g = mode ? i - a.slots : i;
  Tile ta{}, tb{};
  const int kind = resolve_slot<BM, BN, GN>(a, S, L, g % kXcds, g / kXcds, mode, ta, tb);
  int4* e = table + kTableInt4 * i;
  e[0] = make_int4(kind, ta.group, ta.e, ta.row0);
  e[1] = make_int4(ta.M, ta.n0, ta.spl, ta.ks);
  e[2] = make_int4(ta.unit0, tb.group, tb.e, tb.row0);
  e[3] = make_int4(kind == 1 ? tb.M : 0, tb.n0, 0, 0);
}

// One launch plans both GEMMs of the FFN (blockIdx.y: 0 up, 1 down).
template <int BM, int BN, int GN>
__global__ __launch_bounds__(kThreads) void big_plan_kernel(GemmArgs up, GemmArgs down) {
  __shared__ SchedLds L;
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
          if (gelu) y = gelu_erf(y);
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
    if (gelu) y = gelu_erf(y);
    C[(size_t)row * N + col] = (uint16_t)f32_to_bf16(y);
  }
}

// ----------------------------------------------------------------- bf16 MFMA, large tiles

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
  static_assert(BM * BN * 2 <= 2 * STAGE && BN == 256, "C tile in LDS: 512-byte rows");
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
          y0 = gelu_erf_fast(y0);
          y1 = gelu_erf_fast(y1);
        }
        const uint32_t own = cvt_bf16x2(y0, y1);  // (row R(v), row R(v) + 1) of this column
        const uint32_t partner = __builtin_amdgcn_update_dpp(0u, own, 0xB1, 0xF, 0xF, false);
        const uint32_t pair = __builtin_amdgcn_perm(partner, own, sel);
        const int roff = (i * 32 + (v >> 2) * 8 + (v & 3)) * CROWB;
        *reinterpret_cast<uint32_t*>(smem + cbase[j] + roff) = pair;
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
  for (int q = threadIdx.x; q < RR * BN / 2; q += kThreads) {
    const int row = r0 + q / (BN / 2), col = (q % (BN / 2)) * 2;
    if (row >= t.M || col >= nvalid) continue;
    float2 v[kMaxSplit];
#pragma unroll
    for (int ks = 0; ks < kMaxSplit; ++ks)  // all loads first, then the sum in slice order
      if (ks < t.spl)
        v[ks] = *reinterpret_cast<const float2*>(P + (size_t)ks * BM * BN + (size_t)row * BN + col);
    float y0 = 0.0f, y1 = 0.0f;
#pragma unroll
    for (int ks = 0; ks < kMaxSplit; ++ks)
      if (ks < t.spl) {
        y0 += v[ks].x;
        y1 += v[ks].y;
      }
    if (gelu) {
      y0 = gelu_erf_fast(y0);
      y1 = gelu_erf_fast(y1);
    }
    *reinterpret_cast<uint32_t*>(C + (size_t)row * N + col) = pack_bf16x2(y0, y1);
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

// K slices of a small-tile launch. With fewer tiles than CUs (a single token:
// every workgroup would walk all of K alone on a CU of its own) K is split so
// that about 1024 workgroups stream the weights, each slice at least 8 stages
// of the routed K; gemm_small_reduce_kernel sums the slices. Measured on the
// graph-replayed decode layer (H = 4096, E = 128, k = 8, F = 1536 + shared):
// T = 1 FFN 55.1 -> 48.7 us (216 up-projection tiles, 4 slices); at T = 2
// (408 tiles) a 2-way split cost 3 us more than it saved, hence the limit.
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

template <int BM, int BN, int WM, int WN>
hipError_t run_bf16(GemmArgs a, int rows, int E, int nks, hipStream_t s) {
  dim3 grid;
  grid_of<BM, BN>(a, rows, E, grid);
  const unsigned nt = grid.x;
  grid.y = nks;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN>), grid, dim3(kThreads), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nks <= 1) return err;
  hipLaunchKernelGGL((gemm_small_reduce_kernel<BM, BN>), dim3(nt), dim3(kThreads), 0, s, a, nks);
  return hipGetLastError();
}

hipError_t run_gemm(const GemmArgs& a, int rows, int E, bool bf16, bool small_segments,
                    hipStream_t s) {
  if (!bf16) {
    GemmArgs b = a;
    dim3 grid;
    grid_of<64, 64>(b, rows, E, grid);
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(kThreads), 0, s, b);
    return hipGetLastError();
  }
  if (small_segments) {
    // 32x64 tiles: 36 KiB rings, so more workgroups per CU keep weight copies
    // in flight than with 32x128 tiles (measured, graph-replayed decode layer,
    // H = 4096, E = 128, k = 8: FFN at T = 128 640 -> 603 us, T = 16 426 ->
    // 412 us, T = 1 unchanged; a four- or five-stage ring gains nothing more)
    const int nks = a.part != nullptr ? small_splits(a, rows, E) : 1;
    return run_bf16<kSmallBM, kSmallBN, 1, 2>(a, rows, E, nks, s);
  }
  // big tiles: the table was written by big_plan_kernel
  if (a.gelu)
    hipLaunchKernelGGL((gemm_bf16_big_kernel<256, 256, kBigWaves, true>), dim3(a.slots),
                       dim3(kBigWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_bf16_big_kernel<256, 256, kBigWaves, false>), dim3(a.slots),
                       dim3(kBigWaves * 64), 0, s, a);
  hipError_t err = hipGetLastError();
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
    int4* tab = static_cast<int4*>(at(Lo.table));
    for (GemmArgs* a : {&up, &down}) {
      // split K only where every group's K is long (see kSplitMinK)
      const bool long_k = a->routed.K >= kSplitMinK && (a->shared_M == 0 || a->shared.K >= kSplitMinK);
      a->part = long_k ? static_cast<float*>(at(Lo.part)) : nullptr;
      // worst-case tiles rounded up to whole slots of every XCD; a split last
      // round adds at most one round of kSlots per XCD
      dim3 grid;
      grid_of<256, 256>(*a, rows, E, grid);
      a->slots = (int)((grid.x + kXcds - 1) / kXcds * kXcds) +
                 (a->part ? kXcds * kSlots : 0);
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
                             hipStream_t s) {
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
  err = run_gemm(Lo.up, rows, E, bf16, Lo.small_segments, s);
  if (err != hipSuccess) return err;
  return run_gemm(Lo.down, rows, E, bf16, Lo.small_segments, s);
}

}  // namespace moe

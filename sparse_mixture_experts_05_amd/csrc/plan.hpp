// Tile schedule of the large-tile grouped-GEMM launches.
//
// Plain integer arithmetic on per-group tables, compiled twice: into the
// device planner (big_plan_kernel in ffn.hip, which fills the tables with
// parallel scans and resolves one workgroup slot per thread) and into host
// code, where plan_table_serial runs the same functions one slot after the
// other (the planner's coverage checks call it through a small host shim).
// No HIP runtime calls and no device intrinsics appear here.
//
// The groups of a launch are the E routed experts (ragged segments of the
// expert-contiguous buffer, from the dispatch offsets) and, when present, the
// always-on shared expert ("hncyxsy.com Kimi K3 fine-grained MoE" article:
// many small experts plus one shared expert; "lpqz.cn MoE engineering blog"
// section 3.1: one buffer grouped by expert).
#pragma once

#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define MOE_HD __host__ __device__
#else
#define MOE_HD
#endif

namespace moe {
namespace plan {

// Blocked, XCD-aware tile order (large tiles). A group with c rows has
// ceil(c/BM) row tiles; if BM does not divide c the last one is partial (it
// skips the 32-row sub-tiles past the segment end).
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
// kMinSliceStages K stages). A slice writes its fp32 partial tile to the
// workspace; a second launch (mode 1 slots) sums the spl partials of each tail
// tile in slice order and runs the epilogue. The partition depends only on the
// counts, so results repeat bit for bit. Only long K qualifies (every group's
// K at least kSplitMinK): a short tail tile does not repay the partial round
// trip and the extra launch (measured on the fine-grained and heavy-skew layers).
constexpr int kXcds = 8;
constexpr int kSlots = 32;    // CUs per XCD: workgroups one round of an XCD runs
constexpr int kMaxSplit = 8;
constexpr int kMinSliceStages = 32;  // a slice writes a 256 KB partial: keep it worth it
constexpr int kSplitMinK = 8192;
constexpr int kStageK = 64;          // K elements per stage of the GEMM main loop
// GN of the tile order: column tiles per n-block. Measured against 8 (FFN,
// same box, two alternating runs): Mixtral-shaped 2162-2166 -> 2133 us,
// fine-grained 1227-1231 -> 1216 us, heavy-skew unchanged; 16 was 3% slower
// on the Mixtral-shaped layer, 2 1-2% slower on the heavy-skew one.
constexpr int kBlockCols = 4;

// Small segments inside a big-tile launch of the 8-wave kernel. A routed
// segment of at most 32 rows would fill one of the 8 sub-tile rows of a
// 256x256 tile while the tile streams the whole weight panel and copies 256
// (clamped) A rows. Such segments run as 32 x 128 tiles (kSBM x kSBN) instead,
// two per workgroup (one per half of the 8 waves, each with its own LDS ring),
// and their slots are spread evenly through each XCD's sequence among the big
// tiles. Measured on the fine-grained and heavy-skew layers: 1-2% off the FFN;
// a 128-row limit (up to 4 strips re-reading the same weights) was 3% slower
// than none. Not in split-K launches, and not for the shared group (the two
// tiles of a workgroup must have the same K: they meet the same barriers). If
// the launch's slots cannot hold the pairs, every segment takes big tiles.
// The 4-wave kernel takes no pairs (Shape::pairs = 0): with one wave per
// SIMD it would run the two small tiles one after the other, and a 256x256
// tile of a short segment (copy-bound, its MFMAs on empty sub-tiles skipped)
// costs a quarter of the time per column.
constexpr int kSmallRows = 33;
constexpr int kSBM = 32, kSBN = 128;

// Split tail tiles a reduce launch can hold: half a round of every XCD.
constexpr int kReduceSlots = kXcds * kSlots / 2;
constexpr int kEntryInts = 16;  // ints per table entry (four int4)
constexpr int kMaxGroups = 257;  // 256 experts and the shared one

MOE_HD inline int imin(int a, int b) { return a < b ? a : b; }
MOE_HD inline int imax(int a, int b) { return a > b ? a : b; }
MOE_HD inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// What the schedule of one launch depends on.
struct Shape {
  int E;           // routed experts
  int rows;        // rows of the routed buffer (offsets are clamped into it)
  int shared_M;    // rows of the shared group (0: none)
  int routed_N, routed_K, shared_N, shared_K;
  int split;       // 1: the launch may split its last round over K
  int slots;       // workgroups of the launch
  int pairs;       // 1: short segments may run as pairs of small tiles
};

struct Tile {
  int group;  // 0 routed, 1 shared
  int e;      // expert (routed)
  int row0;   // first row of the tile in A / C
  int M;      // valid rows in this tile
  int n0;     // first column
  int spl;    // K slices of this tile (1: the whole K in one workgroup)
  int ks;     // this workgroup's slice
  int unit0;  // partial-tile index of slice 0 (split tiles), else -1
};

// Per-group tables (inclusive scans over groups once complete).
struct Tables {
  int pf[kMaxGroups];    // big tiles by group when short segments take tile pairs
  int pa[kMaxGroups];    // big tiles by group when every segment takes big tiles
  int ps[kMaxGroups];    // short-segment tiles by group
  int goff[kMaxGroups], gcnt[kMaxGroups];  // first row and rows of each group
};

struct Sched {
  const int* pf;     // big-tile scan in use
  int F, CF;         // big tiles in all; per XCD
  int P, CP;         // short-segment pairs in all; per XCD
  int R, tail, spl;  // whole rounds per XCD, tiles of the last round, K slices of those
};

MOE_HD inline int num_groups(const Shape& s) { return s.E + (s.shared_M > 0 ? 1 : 0); }

// A launch splits its last round over K only where every group's K is long.
MOE_HD inline bool split_ok(const Shape& s) {
  return s.routed_K >= kSplitMinK && (s.shared_M == 0 || s.shared_K >= kSplitMinK);
}

// Workgroups of a big-tile launch: the worst-case tile count (sum over experts
// of ceil(count/BM) <= rows/BM + min(E, rows)) rounded up to whole slots of
// every XCD; a split last round adds at most one round of kSlots per XCD.
template <int BM, int BN>
MOE_HD inline int launch_slots(const Shape& s) {
  const long long mt_max = s.rows / BM + imin(s.E, s.rows);
  const long long routed = mt_max * cdiv(s.routed_N, BN);
  const long long shared = s.shared_M > 0 ? (long long)cdiv(s.shared_M, BM) * cdiv(s.shared_N, BN) : 0;
  const long long grid = routed + shared;
  return (int)((grid + kXcds - 1) / kXcds * kXcds) + (s.split ? kXcds * kSlots : 0);
}

// Table entries of group grp before the scans: first row, rows, big tiles
// with and without short-segment pairs, short-segment tiles. Offsets come from
// the dispatch step; clamping keeps every segment inside the buffer even if a
// caller passes inconsistent offsets.
template <int BM, int BN>
MOE_HD inline void group_entry(const Shape& s, const int32_t* offsets, int grp, int& off,
                               int& cnt, int& all, int& big, int& sml) {
  off = cnt = all = big = sml = 0;
  if (grp >= num_groups(s)) return;
  if (grp < s.E) {
    off = imin(imax(offsets[grp], 0), s.rows);
    cnt = imin(imax(offsets[grp + 1], off), s.rows) - off;
  } else {
    off = 0;
    cnt = s.shared_M;
  }
  all = cdiv(cnt, BM) * (grp < s.E ? cdiv(s.routed_N, BN) : cdiv(s.shared_N, BN));
  const bool small = s.pairs && !s.split && grp < s.E && cnt > 0 && cnt < kSmallRows;
  big = small ? 0 : all;
  sml = small ? cdiv(cnt, kSBM) * cdiv(s.routed_N, kSBN) : 0;
}

// The schedule from the completed scans (the same for every workgroup, and
// for every tile a workgroup runs).
MOE_HD inline Sched finish_schedule(const Shape& s, const Tables& L) {
  const int last = num_groups(s) - 1;
  Sched S;
  const int Fs = L.pf[last], Ps = (L.ps[last] + 1) / 2;
  const int CFs = cdiv(Fs, kXcds), CPs = cdiv(Ps, kXcds);
  if (Ps > 0 && kXcds * (CFs + CPs) <= s.slots && CFs + CPs < (1 << 15)) {
    S.pf = L.pf;
    S.F = Fs;
    S.P = Ps;
  } else {
    S.pf = L.pa;
    S.F = L.pa[last];
    S.P = 0;
  }
  S.CF = cdiv(S.F, kXcds);
  S.CP = cdiv(S.P, kXcds);
  S.R = S.CF / kSlots;
  S.tail = S.CF - S.R * kSlots;
  S.spl = 1;
  if (s.split && S.tail > 0 && 2 * S.tail <= kSlots) {
    int ktmin = s.routed_K / kStageK;
    if (s.shared_M > 0) ktmin = imin(ktmin, s.shared_K / kStageK);
    S.spl = imax(1, imin(imin(kSlots / S.tail, kMaxSplit), ktmin / kMinSliceStages));
  }
  return S;
}

// The first entry of an inclusive scan over groups [0, ng) above q.
MOE_HD inline int scan_find(const int* scan, int ng, int q) {
  int lo = 0, hi = ng - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (scan[mid] > q) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// Short-segment tile u of the launch (u < number of short-segment tiles).
MOE_HD inline void small_tile_of(const Shape& s, const Tables& L, int u, Tile& t) {
  const int grp = scan_find(L.ps, s.E, u);
  const int li = u - (grp ? L.ps[grp - 1] : 0);
  const int c = L.gcnt[grp];
  const int nrs = cdiv(c, kSBM);  // row strips of the segment
  const int r = li % nrs;
  t.group = 0;
  t.e = grp;
  t.row0 = L.goff[grp] + r * kSBM;
  t.M = imin(kSBM, c - r * kSBM);
  t.n0 = (li / nrs) * kSBN;
  t.spl = 1;
  t.ks = 0;
  t.unit0 = -1;
}

// Slot `slot` on XCD x. mode 0: the launch's work, kind 0 = one big tile (or
// K slice of a split tail tile) in ta, kind 1 = a pair of short-segment tiles
// (ta, and tb unless tb.M == 0); mode 1: the split tail tile number `slot` to
// reduce (kind 0). Returns -1 if the slot holds nothing.
// An XCD runs CF big-tile slots and CP pair slots; pair slots sit at the
// positions q where floor((q + 1) * CP / n) steps (n = CF + CP), evenly spread.
template <int BM, int BN, int GN>
MOE_HD inline int resolve_slot(const Shape& s, const Sched& S, const Tables& L, int x, int slot,
                               int mode, Tile& ta, Tile& tb) {
  const int ng = num_groups(s);
  const int ntr = cdiv(s.routed_N, BN);
  const int nts = cdiv(s.shared_N, BN);
  const int F = S.F, CF = S.CF, R = S.R, tail = S.tail, spl = S.spl;
  int ks = 0, unit0 = -1;
  tb.M = 0;
  if (mode == 0) {
    if (S.CP > 0) {  // pairs (never with split K, whose slices sit past CF)
      const int n = CF + S.CP;
      if (slot >= n) return -1;
      // slot < n < 2^15 and CP < 2^15 (pairs only then): the products fit 32 bits
      const int pb = (int)((unsigned)(slot * S.CP) / (unsigned)n);
      if ((int)((unsigned)((slot + 1) * S.CP) / (unsigned)n) > pb) {  // a pair slot
        const int p = pb * kXcds + x;
        if (p >= S.P) return -1;
        const int nsm = L.ps[s.E - 1];
        small_tile_of(s, L, 2 * p, ta);
        if (2 * p + 1 < nsm) small_tile_of(s, L, 2 * p + 1, tb);
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
  const int mt_g = cdiv(c, BM);  // row tiles of the group, the last one maybe partial
  const int nt_g = grp < s.E ? ntr : nts;
  const int local = q - excl;
  const int blk = local / (mt_g * GN);
  const int w = imin(GN, nt_g - blk * GN);
  const int li = local - blk * mt_g * GN;
  ta.row0 = o + (li / w) * BM;
  ta.M = imin(BM, c - (li / w) * BM);
  ta.n0 = (blk * GN + li % w) * BN;
  ta.group = grp < s.E ? 0 : 1;
  ta.e = grp < s.E ? grp : 0;
  ta.spl = unit0 >= 0 ? spl : 1;
  ta.ks = ks;
  ta.unit0 = unit0;
  return 0;
}

// One table entry, 16 ints: {kind, group a, expert a, row0 a}, {M a, n0 a,
// spl, ks}, {unit0, group b, expert b, row0 b}, {M b, n0 b, 0, 0}
// (kind -1: nothing; 0: a big tile in a; 1: short-segment tiles a and b,
// b absent if M b = 0).
MOE_HD inline void encode_entry(int kind, const Tile& ta, const Tile& tb, int* e) {
  e[0] = kind, e[1] = ta.group, e[2] = ta.e, e[3] = ta.row0;
  e[4] = ta.M, e[5] = ta.n0, e[6] = ta.spl, e[7] = ta.ks;
  e[8] = ta.unit0, e[9] = tb.group, e[10] = tb.e, e[11] = tb.row0;
  e[12] = kind == 1 ? tb.M : 0, e[13] = tb.n0, e[14] = 0, e[15] = 0;
}

// The whole table of a launch, one slot after the other: slots [0, s.slots)
// of the GEMM launch (workgroup g: slot g / 8 on XCD g % 8), then
// kReduceSlots of its split-K reduce. table holds
// (s.slots + kReduceSlots) * kEntryInts ints. The device planner computes
// the same entries with the tables scanned in parallel.
template <int BM, int BN, int GN>
inline void plan_table_serial(const Shape& s, const int32_t* offsets, int* table) {
  static Tables L;  // large: keep it off the stack
  int run_a = 0, run_f = 0, run_s = 0;
  for (int g = 0; g < kMaxGroups; ++g) {
    int off, cnt, all, big, sml;
    group_entry<BM, BN>(s, offsets, g, off, cnt, all, big, sml);
    L.goff[g] = off;
    L.gcnt[g] = cnt;
    L.pa[g] = run_a += all;
    L.pf[g] = run_f += big;
    L.ps[g] = run_s += sml;
  }
  const Sched S = finish_schedule(s, L);
  for (int i = 0; i < s.slots + kReduceSlots; ++i) {
    const int mode = i < s.slots ? 0 : 1;
    const int g = mode ? i - s.slots : i;
    Tile ta{}, tb{};
    const int kind = resolve_slot<BM, BN, GN>(s, S, L, g % kXcds, g / kXcds, mode, ta, tb);
    encode_entry(kind, ta, tb, table + (size_t)kEntryInts * i);
  }
}

}  // namespace plan
}  // namespace moe

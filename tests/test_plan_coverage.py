"""Coverage of the big-tile schedule of the grouped GEMM (host logic check).

The planner of csrc/ffn.hip (big_schedule, resolve_slot, small_tile_of) runs on
the device; this file transcribes its integer arithmetic step for step and
checks, over random expert-count vectors, shapes and both launch kinds (split
K in the last round; small-segment pairs), that the workgroup slots cover every
32-row x 128-column block of every segment and of the shared group exactly once, each split
tile in all its K slices, that small tiles stay inside their segments, and
that the reduce slots are exactly the split tail tiles. It must follow the
device code when that changes; the GPU tests check the device code itself.
"""
import numpy as np
# constants of ffn.hip: XCDs, CUs per XCD, split limits, small-segment rows, tile shapes, n-block
kX, kSlots, kMaxSplit, kMinSlice, kSmallRows, kSBM, kSBN, BM, BN, GN = 8, 32, 8, 32, 33, 32, 128, 256, 256, 4
kReduce = kX * kSlots // 2
def cdiv(a, b): return (a + b - 1) // b
def sched(counts, Nr, Kr, shared_M, Ns, Ks, part, slots):
    E = len(counts); ng = E + (1 if shared_M > 0 else 0)
    off = np.concatenate([[0], np.cumsum(counts)])
    goff = list(off[:E]) + ([0] if shared_M else []); gcnt = list(counts) + ([shared_M] if shared_M else [])
    ntr, nts, nsr = cdiv(Nr, BN), cdiv(Ns, BN), cdiv(Nr, kSBN)
    small_ok = part is None
    pa, pf, ps = [], [], []
    for g in range(ng):
        c = gcnt[g]; allt = cdiv(c, BM) * (ntr if g < E else nts)
        sm = small_ok and g < E and 0 < c < kSmallRows
        pa.append(allt); pf.append(0 if sm else allt); ps.append(cdiv(c, kSBM) * nsr if sm else 0)
    pa, pf, ps = np.cumsum(pa), np.cumsum(pf), np.cumsum(ps)
    Fs, Ps = pf[-1], (ps[E - 1] + 1) // 2
    if Ps > 0 and kX * (cdiv(Fs, kX) + cdiv(Ps, kX)) <= slots and cdiv(Fs, kX) + cdiv(Ps, kX) < (1 << 15): use, F, P = pf, Fs, Ps
    else: use, F, P = pa, pa[-1], 0
    CF, CP = cdiv(F, kX), cdiv(P, kX)
    R, tail = CF // kSlots, CF - (CF // kSlots) * kSlots
    spl = 1
    if part is not None and tail > 0 and 2 * tail <= kSlots:
        ktmin = Kr // 64
        if shared_M > 0: ktmin = min(ktmin, Ks // 64)
        spl = max(1, min(min(kSlots // tail, kMaxSplit), ktmin // kMinSlice))
    return dict(E=E, ng=ng, goff=goff, gcnt=gcnt, use=use, ps=ps, F=F, P=P, CF=CF, CP=CP, R=R, tail=tail, spl=spl, ntr=ntr, nts=nts)
def find(scan, n, q):
    lo, hi = 0, n - 1
    while lo < hi:
        mid = (lo + hi) // 2
        if scan[mid] > q: hi = mid
        else: lo = mid + 1
    return lo
def small_of(S, u):
    g = find(S["ps"], S["E"], u); li = u - (S["ps"][g - 1] if g else 0); c = S["gcnt"][g]; nrs = cdiv(c, kSBM)
    r = li % nrs
    return ("s", g, S["goff"][g] + r * kSBM, min(kSBM, c - r * kSBM), (li // nrs) * kSBN)
def resolve(S, x, slot, mode):
    CF, R, tail, spl = S["CF"], S["R"], S["tail"], S["spl"]; ks, unit0 = 0, -1
    if mode == 0:
        if S["CP"] > 0:
            n = CF + S["CP"]
            if slot >= n: return None
            pb = slot * S["CP"] // n
            if (slot + 1) * S["CP"] // n > pb:
                p = pb * kX + x
                if p >= S["P"]: return None
                nsm = S["ps"][S["E"] - 1]
                a = small_of(S, 2 * p); b = small_of(S, 2 * p + 1) if 2 * p + 1 < nsm else None
                return ("pair", a, b)
            slot -= pb
        if spl > 1 and slot >= R * kSlots:
            u = slot - R * kSlots
            if u >= tail * spl: return None
            tt = u // spl; ks = u - tt * spl; slot = R * kSlots + tt; unit0 = x * kSlots + tt * spl
    else:
        if spl <= 1 or slot >= tail: return None
        unit0 = x * kSlots + slot * spl; slot = R * kSlots + slot
    if slot >= CF: return None
    q = x * CF + slot
    if q >= S["F"]: return None
    use = S["use"]; g = find(use, S["ng"], q); excl = use[g - 1] if g else 0
    o, c = S["goff"][g], S["gcnt"][g]; mt = cdiv(c, BM); nt = S["ntr"] if g < S["E"] else S["nts"]
    local = q - excl; blk = local // (mt * GN); w = min(GN, nt - blk * GN); li = local - blk * mt * GN
    return ("big", g, o + (li // w) * BM, min(BM, c - (li // w) * BM), (blk * GN + li % w) * BN, spl if unit0 >= 0 else 1, ks, unit0)
def check(counts, Nr, Kr, shared_M, Ns, Ks, part):
    E = len(counts); rows = int(sum(counts))
    grid = (rows // BM + min(E, rows)) * cdiv(Nr, BN) + (cdiv(shared_M, BM) * cdiv(Ns, BN) if shared_M else 0)
    slots = cdiv(grid, kX) * kX + (kX * kSlots if part else 0)
    S = sched(counts, Nr, Kr, shared_M, Ns, Ks, part, slots)
    cover = {}  # (group, row, col) element blocks -> list of k slices
    red = set()
    for g in range(slots):
        r = resolve(S, g % kX, g // kX, 0)
        if r is None: continue
        if r[0] == "pair":
            for t in r[1:]:
                if t is None: continue
                _, gr, row0, M, n0 = t
                assert 0 < M <= kSBM and row0 >= S["goff"][gr] and row0 + M <= S["goff"][gr] + S["gcnt"][gr]
                for rr in range(row0, row0 + M, 32):
                    for cc in range(n0, min(n0 + kSBN, Nr), 128):
                        cover.setdefault((gr, rr, cc), []).append((0, 1))
        else:
            _, gr, row0, M, n0, sp, ks, unit0 = r
            N = Nr if gr < E else Ns
            for rr in range(row0, row0 + M, 32):
                for cc in range(n0, min(n0 + BN, N), 128):
                    cover.setdefault((gr, rr, cc), []).append((ks, sp))
            if unit0 >= 0: red.add(unit0)
    # reduce slots: exactly the split tail tiles, each once
    seen = set()
    for i in range(kReduce):
        r = resolve(S, i % kX, i // kX, 1)
        if r is not None:
            assert r[7] in red and r[7] not in seen
            seen.add(r[7])
    assert seen == red
    expect = set()
    for gr in range(E):
        base = S["goff"][gr]; c = S["gcnt"][gr]
        if c == 0: continue
        step = kSBM if (S["P"] > 0 and 0 < c < kSmallRows) else BM
        for t0 in range(base, base + c, step):
            for rr in range(t0, min(t0 + step, base + c), 32):
                for cc in range(0, Nr, 128): expect.add((gr, rr, cc))
    if shared_M:
        for rr in range(0, shared_M, 32):
            for cc in range(0, Ns, 128): expect.add((E, rr, cc))
    assert set(cover) == expect, (len(set(cover) ^ expect))
    for k, v in cover.items():
        sp = v[0][1]
        assert sorted(x[0] for x in v) == list(range(sp)), (k, v)
    return S["P"], S["spl"]


def test_schedule_covers_every_block_once():
    rng = np.random.default_rng(0)
    stats = {"pairs": 0, "split": 0}
    for trial in range(120):
        E = int(rng.choice([1, 4, 8, 16, 64, 128, 256]))
        rows = int(rng.integers(64 * E, 64 * E * 3 + 1))
        p = rng.dirichlet(np.full(E, rng.choice([0.05, 0.3, 1.0, 5.0])))
        counts = rng.multinomial(rows, p)
        H = int(rng.choice([256, 1024, 4096]))
        F = int(rng.choice([512, 1536, 8192, 14336]))
        Fs = int(rng.choice([0, F]))
        T = rows // max(1, int(rng.choice([1, 2, 8])))
        for (Nr, Kr, Ns, Ks) in [(F, H, Fs, H), (H, F, H, Fs)]:
            part = "p" if (Kr >= 8192 and (Fs == 0 or Ks >= 8192)) else None
            P, spl = check(counts, Nr, Kr, T if Fs else 0, Ns, Ks, part)
            stats["pairs"] += P > 0
            stats["split"] += spl > 1
    # both launch kinds were exercised
    assert stats["pairs"] > 20 and stats["split"] > 20, stats

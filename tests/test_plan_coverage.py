"""Coverage of the big-tile schedule of the grouped GEMM (host check, no GPU).

The planner's arithmetic lives in the library's csrc/plan.hpp; the device
planner (big_plan_kernel) and this check run the same functions. The test
compiles plan.hpp with a small host shim (tests/plan_host.cpp) and checks,
over random expert-count vectors, shapes and both launch kinds (split K in the
last round; short-segment pairs), the table it writes:
  * every 32-row x 128-column block of every segment and of the shared group
    is computed exactly once (each split tile in all of its K slices),
  * short-segment tiles stay inside their segments, big tiles inside the
    buffer and the column range,
  * the reduce slots are exactly the split tail tiles, each once.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_mixture_experts_05_amd", "csrc")
BM = BN = 256
SBM, SBN = 32, 128  # short-segment tiles (plan.hpp kSBM, kSBN)


@pytest.fixture(scope="module")
def planner(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("plan") / "plan_host.so")
    cmd = ["g++", "-O2", "-std=c++17", "-shared", "-fPIC", f"-I{CSRC}",
           os.path.join(ROOT, "tests", "plan_host.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    L = ctypes.CDLL(out)
    i, p = ctypes.c_int, ctypes.c_void_p
    L.moe_plan_slots.restype = i
    L.moe_plan_slots.argtypes = [i] * 8 + [ctypes.POINTER(i)]
    L.moe_plan_table.restype = None
    L.moe_plan_table.argtypes = [p] + [i] * 10 + [p]
    return L


def plan(L, counts, Nr, Kr, shared_M, Ns, Ks, pairs=1):
    """(table [slots + reduce, 16], slots, split) of one launch."""
    E = len(counts)
    rows = int(sum(counts))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    split = ctypes.c_int(0)
    slots = L.moe_plan_slots(E, rows, shared_M, Nr, Kr, Ns, Ks, pairs, ctypes.byref(split))
    n = slots + L.moe_plan_reduce_slots()
    table = np.full((n, L.moe_plan_entry_ints()), -7, dtype=np.int32)
    L.moe_plan_table(offsets.ctypes.data, E, rows, shared_M, Nr, Kr, Ns, Ks, split.value, slots,
                     pairs, table.ctypes.data)
    return table, slots, split.value


def check(L, counts, Nr, Kr, shared_M, Ns, Ks, pairs=1):
    E = len(counts)
    goff = list(np.concatenate([[0], np.cumsum(counts)])[:E]) + [0]
    gcnt = list(counts) + [shared_M]
    table, slots, split = plan(L, counts, Nr, Kr, shared_M, Ns, Ks, pairs)
    cover = {}  # (group, row, col) blocks -> list of (k slice, slices)
    red = set()
    npairs = 0
    for g in range(slots):
        e = table[g]
        kind = e[0]
        if kind < 0:
            continue
        if kind == 1:
            npairs += 1
            assert not split and pairs  # no pairs in split-K launches or when not allowed
            for (grp, ex, row0, M, n0) in [(e[1], e[2], e[3], e[4], e[5]),
                                           (e[9], e[10], e[11], e[12], e[13])]:
                if M == 0:
                    continue
                assert grp == 0 and 0 < M <= SBM
                assert goff[ex] <= row0 and row0 + M <= goff[ex] + gcnt[ex]
                assert gcnt[ex] < 33  # only short segments take small tiles
                for rr in range(row0, row0 + M, 32):
                    for cc in range(n0, min(n0 + SBN, Nr), 128):
                        cover.setdefault((ex, rr, cc), []).append((0, 1))
            continue
        assert kind == 0
        grp, ex, row0, M, n0, spl, ks, unit0 = e[1:9]
        gi = ex if grp == 0 else E
        N = Nr if grp == 0 else Ns
        assert 0 < M <= BM and goff[gi] <= row0 and row0 + M <= goff[gi] + gcnt[gi]
        assert 0 <= n0 < N and n0 % BN == 0
        assert (spl == 1 and ks == 0 and unit0 == -1) or (split and 0 <= ks < spl and unit0 >= 0)
        for rr in range(row0, row0 + M, 32):
            for cc in range(n0, min(n0 + BN, N), 128):
                cover.setdefault((gi, rr, cc), []).append((ks, spl))
        if unit0 >= 0:
            red.add(int(unit0))
    # reduce slots: exactly the split tail tiles, each once
    seen = set()
    for e in table[slots:]:
        if e[0] < 0:
            continue
        assert e[0] == 0 and e[6] > 1
        assert int(e[8]) in red and int(e[8]) not in seen
        seen.add(int(e[8]))
    assert seen == red
    expect = set()
    for gi in range(E + (1 if shared_M else 0)):
        N = Nr if gi < E else Ns
        for rr in range(goff[gi], goff[gi] + gcnt[gi], 32):
            for cc in range(0, N, 128):
                expect.add((gi, rr, cc))
    assert set(cover) == expect, len(set(cover) ^ expect)
    for key, v in cover.items():
        sp = v[0][1]
        assert sorted(x[0] for x in v) == list(range(sp)), (key, v)
    return npairs, split and any(table[g][6] > 1 for g in range(slots) if table[g][0] == 0)


def test_schedule_covers_every_block_once(planner):
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
            for allow in (1, 0):  # the 8-wave kernel's plan, then the 4-wave kernel's
                pairs, split = check(planner, counts, Nr, Kr, T if Fs else 0, Ns, Ks, allow)
                stats["pairs"] += pairs > 0
                stats["split"] += bool(split)
                assert allow or pairs == 0
    # both launch kinds were exercised
    assert stats["pairs"] > 20 and stats["split"] > 20, stats


def test_schedule_of_the_workload_shapes(planner):
    """The three big-tile workloads with their expected routing shapes: the
    Mixtral-shaped down projection splits its last round; the fine-grained
    layer's short segments run in pairs; E = 256 with a shared expert (257
    groups) is covered too."""
    rng = np.random.default_rng(1)
    mix = np.array([982, 1067, 1010, 1040, 1001, 1023, 1050, 1019])
    assert check(planner, mix, 4096, 14336, 0, 4096, 14336)[1]   # split tail
    assert not check(planner, mix, 14336, 4096, 0, 14336, 4096)[1]
    fg = rng.multinomial(32768, rng.dirichlet(np.full(128, 0.05)))
    assert check(planner, fg, 1536, 4096, 4096, 1536, 4096)[0] > 0  # pairs
    assert check(planner, fg, 1536, 4096, 4096, 1536, 4096, pairs=0)[0] == 0
    check(planner, fg, 4096, 1536, 4096, 4096, 1536)
    hs = rng.multinomial(131072, rng.dirichlet(np.full(256, 0.05)))
    check(planner, hs, 1024, 4096, 0, 1024, 4096)
    check(planner, hs, 4096, 1024, 16384, 4096, 1024)               # 257 groups
    # edge cases: one row in all, everything in one expert, empty experts
    check(planner, np.array([1]), 512, 256, 0, 512, 256)
    check(planner, np.array([0, 0, 5000, 0]), 4096, 8192, 0, 4096, 8192)
    check(planner, np.array([0] * 255 + [300]), 1024, 4096, 300, 1024, 4096)

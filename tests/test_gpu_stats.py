"""moe_load_stats through the C ABI on count vectors picked for the kernel's
two ways of ranking the counts, against the oracle's statistics.

The kernel ranks count c_e among all counts (ties broken by expert id) either
by comparing packed keys (c << 8 | id), when every count lies in [0, 2^24),
or by comparing counts and ids separately otherwise. Counts from a layer
never reach 2^24, so the cases below also feed counts that do, and counts on
both sides of that boundary; ties exercise the id order. T and k only set
the capacity and the drop rate, so the counts need not sum to T*k here.
Every field must equal the oracle's bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_mixture_experts_05_amd import moe_load_stats

pytestmark = pytest.mark.gpu

KEYS = ["num_tokens", "assignments", "capacity", "max_load", "min_load", "dropped",
        "num_stragglers", "gini_num", "gini_den", "gini", "load_skew_ratio", "drop_rate",
        "overflow", "straggler_ids"]


def _cases():
    rng = np.random.default_rng([5, 24])
    # name, counts, T, k, cf
    yield "ties_E256", np.repeat(np.arange(16), 16)[rng.permutation(256)] * 3, 4096, 8, 1.25
    yield "all_equal_E200", np.full(200, 77), 1000, 8, 1.25
    yield "zeros_E128", np.zeros(128, dtype=np.int64), 4096, 8, 1.25
    yield "below_2^24_E64", rng.integers(2 ** 24 - 40, 2 ** 24, size=64), 1 << 20, 8, 1.25
    yield "at_2^24_E64", np.concatenate([[2 ** 24], rng.integers(0, 100, size=63)]), 1 << 20, 8, 1.25
    yield "near_int32_E256", rng.integers(2 ** 31 - 1000, 2 ** 31 - 1, size=256), 1 << 24, 8, 1.25
    yield "near_int32_ties_E33", np.repeat([2 ** 31 - 2, 2 ** 31 - 5, 3], 11), 1 << 24, 2, 1.0
    yield "E1_big", np.array([2 ** 30]), 1 << 28, 1, 1.25


CASES = list(_cases())


@pytest.mark.parametrize("name,counts,T,k,cf", CASES, ids=[c[0] for c in CASES])
def test_load_stats_rank_paths(name, counts, T, k, cf):
    E = counts.size
    print(f"\n[gpu] load_stats {name}: E={E} T={T} k={k} max={int(counts.max())}", flush=True)
    c = torch.from_numpy(counts.astype(np.int32)).cuda()
    got = moe_load_stats(c, T, k, cf)
    ref = oracle.load_stats(counts.astype(np.int64), T, k, cf)
    for key in KEYS:
        assert got[key] == ref[key], f"{key}: {got[key]} != {ref[key]}"
    assert all(v == -1 for v in got["straggler_tail"]), "straggler list tail not -1"

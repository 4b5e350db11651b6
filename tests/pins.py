"""Pins of the CPU oracle against what the pages and mathematics fix.

Each check reads the oracle through the module object at call time, so the
mutation tests can plant a mistake in the oracle and see a check fail.
Kinds of pin: closed forms on designed inputs, hand-worked fixtures
(tests/golden/), brute force on tiny inputs, invariants, and special cases
that reduce to an independent library routine (scipy/torch).
"""
from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import scipy.special
import torch

import oracle.moe_oracle as O
from synth import CONFIGS, DECODE_TOKENS, get_config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PHI_1 = 0.8413447460685429   # standard normal CDF at 1 (textbook table value)


def _rng(*key):
    return np.random.default_rng([12345, *key])


# ------------------------------------------------------------------ route

def check_route_onehot_closed_form():
    """x = one-hot e_h, Wg[:, h] = 0.1*e: scores are 0.1*e; top-k is E-1, E-2, ...
    and w_j = r^j (1-r)/(1-r^k) with r = exp(-0.1) (renormalised softmax)."""
    E, H, k = 8, 16, 3
    wg = np.zeros((E, H))
    h = 5
    wg[:, h] = 0.1 * np.arange(E)
    wg[:, (h + 1) % H] = -0.1 * np.arange(E)  # a different column: must not matter
    x = np.zeros((2, H))
    x[:, h] = 1.0
    idx, w, _, _ = O.route(x, wg, None, k)
    assert idx.tolist() == [[7, 6, 5], [7, 6, 5]], idx
    r = math.exp(-0.1)
    want = [r ** j * (1 - r) / (1 - r ** k) for j in range(k)]
    np.testing.assert_allclose(w[0], want, rtol=0, atol=1e-7)


def check_route_bias_closed_form():
    """x = 0 so the scores are the bias. b_e = ln(e+1): p_e is proportional to e+1,
    the top-k are E-1..E-k and w_j = (E-j) / sum_{i<k} (E-i)."""
    E, H, k = 6, 4, 4
    bias = np.log(np.arange(1, E + 1)).astype(np.float32)
    x = np.zeros((3, H))
    wg = _rng(1).standard_normal((E, H))
    idx, w, _, _ = O.route(x, wg, bias, k)
    assert idx[0].tolist() == [5, 4, 3, 2]
    den = sum(E - i for i in range(k))
    np.testing.assert_allclose(w[0], [(E - j) / den for j in range(k)], atol=2e-7)


def check_route_shift_invariance():
    """Adding one constant to every score leaves ids and weights unchanged."""
    x = _rng(2).standard_normal((32, 16))
    wg = _rng(3).standard_normal((8, 16))
    i0, w0, _, _ = O.route(x, wg, None, 3)
    i1, w1, _, _ = O.route(x, wg, np.full(8, 7.25, dtype=np.float32), 3)
    assert (i0 == i1).all()
    np.testing.assert_allclose(w0, w1, atol=1e-6)


def check_route_bias_moves_weights():
    """The bias is inside the softmax: it changes the weights of the same selection."""
    x = np.zeros((1, 4))
    wg = np.zeros((4, 4))
    bias = np.array([1.0, 0.0, 0.5, -3.0], dtype=np.float32)
    idx, w, _, _ = O.route(x, wg, bias, 2)
    assert idx[0].tolist() == [0, 2]
    np.testing.assert_allclose(w[0], [1 / (1 + math.exp(-0.5)), math.exp(-0.5) / (1 + math.exp(-0.5))],
                               atol=1e-7)


def check_route_k_equals_E_is_softmax():
    """k = E: the renormalised weights are the full softmax (scipy), ids sort the scores."""
    x = _rng(4).standard_normal((20, 12))
    wg = _rng(5).standard_normal((6, 12))
    idx, w, _, _ = O.route(x, wg, None, 6)
    sm = scipy.special.softmax(x @ wg.T, axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(sm, idx.astype(np.int64), 1), atol=1e-7)
    assert (np.diff(np.take_along_axis(sm, idx.astype(np.int64), 1), axis=1) <= 0).all()


def check_route_brute_force():
    """Tiny inputs: the chosen set maximises the score sum over all C(E, k) subsets,
    and the order is the descending stable sort of the scores."""
    for E, k in [(2, 1), (4, 2), (5, 3), (8, 3), (8, 1)]:
        H = 8
        x = _rng(6, E, k).standard_normal((16, H))
        wg = _rng(7, E, k).standard_normal((E, H))
        b = _rng(8, E, k).standard_normal(E).astype(np.float32)
        idx, w, s, _ = O.route(x, wg, b, k)
        s_ref = x @ wg.T + b.astype(np.float64)
        for t in range(16):
            best = max(itertools.combinations(range(E), k), key=lambda c: sum(s_ref[t, list(c)]))
            assert sorted(idx[t].tolist()) == sorted(best)
            assert idx[t].tolist() == np.argsort(-s_ref[t], kind="stable")[:k].tolist()
        np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-6)


def check_route_tie_lower_id():
    """Equal scores: the lower expert id comes first."""
    x = np.zeros((1, 4))
    wg = np.zeros((5, 4))
    idx, w, _, _ = O.route(x, wg, None, 3)
    assert idx[0].tolist() == [0, 1, 2]
    np.testing.assert_allclose(w[0], [1 / 3] * 3, atol=1e-7)


def check_route_matches_page_listing_in_torch():
    """The Kimi K3 router listing executed with torch ops (gate Linear without
    bias, softmax, topk, divide by the sum), in float64, on generic inputs."""
    x = _rng(9).standard_normal((64, 32))
    wg = _rng(10).standard_normal((16, 32))
    idx, w, _, _ = O.route(x, wg, None, 4)
    xt, wt = torch.from_numpy(x), torch.from_numpy(wg)
    gate = torch.nn.functional.linear(xt, wt)
    sc = torch.softmax(gate, dim=-1)
    tw, ti = torch.topk(sc, 4, dim=-1)
    tw = tw / tw.sum(dim=-1, keepdim=True)
    assert (ti.numpy() == idx).all()
    np.testing.assert_allclose(w, tw.numpy(), atol=1e-7)


# ------------------------------------------------------------------ dispatch

def check_dispatch_hand_fixture():
    cases = json.load(open(os.path.join(GOLDEN, "dispatch_stats_hand.json")))["cases"]
    for c in cases:
        T, k, E = c["T"], c["k"], c["E"]
        x = np.arange(T * 3, dtype=np.float32).reshape(T, 3)
        counts, offsets, perm, inv, xs = O.dispatch(np.array(c["idx"]), x, E)
        assert counts.tolist() == c["counts"]
        assert offsets.tolist() == c["offsets"]
        assert perm.tolist() == c["perm"]
        assert inv.tolist() == c["inv"]
        assert (xs == x[c["xs_tokens"]]).all()


def _random_topk(T, E, k, seed):
    r = _rng(11, seed)
    return np.stack([r.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


def check_dispatch_invariants():
    for T, E, k in [(1, 1, 1), (7, 3, 2), (100, 8, 2), (257, 64, 8), (50, 256, 8)]:
        idx = _random_topk(T, E, k, T + E)
        x = _rng(12, T).standard_normal((T, 4)).astype(np.float32)
        counts, offsets, perm, inv, xs = O.dispatch(idx, x, E)
        flat = idx.reshape(-1)
        assert (counts == np.bincount(flat, minlength=E)).all()
        assert offsets[0] == 0 and offsets[-1] == T * k
        assert (np.diff(offsets) == counts).all()
        assert sorted(perm.tolist()) == list(range(T * k))
        assert (inv[perm] == np.arange(T * k)).all()
        assert (perm == np.argsort(flat, kind="stable")).all()
        for e in range(E):
            seg = perm[offsets[e]:offsets[e + 1]]
            assert (flat[seg] == e).all()
            assert (np.diff(seg // k) > 0).all()
        assert (xs == x[perm // k]).all()


# ------------------------------------------------------------------ expert FFN

def check_gelu_values():
    g = O.gelu_erf(np.array([0.0, 1.0, -1.0, 2.0, -2.0, 40.0, -40.0]))
    assert g[0] == 0.0
    np.testing.assert_allclose(g[1], PHI_1, rtol=1e-15)
    np.testing.assert_allclose(g[2], PHI_1 - 1.0, rtol=1e-14)
    np.testing.assert_allclose(g[3] - g[4], 2.0, rtol=1e-15)
    assert g[5] == 40.0 and g[6] == 0.0
    a = _rng(13).standard_normal(1000) * 3
    np.testing.assert_allclose(O.gelu_erf(a) - O.gelu_erf(-a), a, atol=1e-14)
    # the erf form, not the tanh approximation (they differ by ~1.5e-4 at a = 1)
    ref = np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in a])
    np.testing.assert_allclose(O.gelu_erf(a), ref, rtol=1e-13, atol=1e-15)


def check_expert_ffn_permutation_closed_form():
    """W1 = [P; 2P] (F = 2H), W2 = [Q, 0]: y = Q gelu(P x), i.e. y[i] = gelu(x[pi[qi[i]]])."""
    H = 8
    pi = _rng(14).permutation(H)
    qi = _rng(15).permutation(H)
    P = np.zeros((H, H)); P[np.arange(H), pi] = 1.0
    Q = np.zeros((H, H)); Q[np.arange(H), qi] = 1.0
    w1 = np.vstack([P, 2 * P])
    w2 = np.hstack([Q, np.zeros((H, H))])
    x = _rng(16).standard_normal((5, H))
    y = O.expert_ffn(x, w1, w2)
    want = np.empty_like(x)
    for i in range(H):
        v = x[:, pi[qi[i]]]
        want[:, i] = [0.5 * a * (1 + math.erf(a / math.sqrt(2))) for a in v]
    np.testing.assert_allclose(y, want, rtol=1e-14, atol=1e-15)


def _torch_ffn(x, w1, w2):
    xt = torch.from_numpy(np.asarray(x, dtype=np.float64))
    a = torch.nn.functional.linear(xt, torch.from_numpy(np.asarray(w1, dtype=np.float64)))
    g = torch.nn.functional.gelu(a, approximate="none")
    return torch.nn.functional.linear(g, torch.from_numpy(np.asarray(w2, dtype=np.float64))).numpy()


def _small_layer(T=24, H=16, E=4, F=32, Fs=0, seed=0, same_experts=False):
    r = _rng(17, seed)
    L = dict(x=r.standard_normal((T, H)).astype(np.float32),
             wg=(r.standard_normal((E, H)) / math.sqrt(H)).astype(np.float32), bias=None)
    if same_experts:
        w1 = np.repeat((r.standard_normal((1, F, H)) / math.sqrt(H)), E, 0)
        w2 = np.repeat((r.standard_normal((1, H, F)) / math.sqrt(F)), E, 0)
    else:
        w1 = r.standard_normal((E, F, H)) / math.sqrt(H)
        w2 = r.standard_normal((E, H, F)) / math.sqrt(F)
    L["w1"], L["w2"] = w1.astype(np.float32), w2.astype(np.float32)
    L["ws1"] = (r.standard_normal((Fs, H)) / math.sqrt(H)).astype(np.float32) if Fs else None
    L["ws2"] = (r.standard_normal((H, Fs)) / math.sqrt(Fs)).astype(np.float32) if Fs else None
    return L


def check_layer_single_expert_is_dense_ffn():
    """E = 1, k = 1: the layer is one dense FFN (torch Linear + exact GeLU)."""
    L = _small_layer(E=1)
    r = O.layer(L, 1)
    assert (r["idx"] == 0).all() and (r["w"] == 1.0).all()
    np.testing.assert_allclose(r["out"], _torch_ffn(L["x"], L["w1"][0], L["w2"][0]), rtol=1e-12, atol=1e-13)


def check_layer_identical_experts():
    """All experts equal: the weights sum to 1, so routing cannot change the output."""
    L = _small_layer(E=6, same_experts=True)
    r = O.layer(L, 3)
    np.testing.assert_allclose(r["out"], _torch_ffn(L["x"], L["w1"][0], L["w2"][0]), rtol=1e-6, atol=1e-7)


def check_layer_scaled_experts_closed_form():
    """W2[e] = (e+1) W2[0] and W1[e] = W1[0]: out = (sum_j w_j (idx_j + 1)) FFN_0(x)."""
    L = _small_layer(E=5, same_experts=True)
    L["w2"] = np.stack([(e + 1) * L["w2"][0].astype(np.float64) for e in range(5)])  # exact scaling
    r = O.layer(L, 2)
    scale = (r["w"].astype(np.float64) * (r["idx"] + 1)).sum(axis=1)
    np.testing.assert_allclose(r["out"], scale[:, None] * _torch_ffn(L["x"], L["w1"][0], L["w2"][0]),
                               rtol=1e-12, atol=1e-12)


def check_layer_shared_expert_is_additive():
    L = _small_layer(E=4, Fs=24)
    with_shared = O.layer(L, 2)["out"]
    L2 = dict(L, ws1=None, ws2=None)
    without = O.layer(L2, 2)["out"]
    np.testing.assert_allclose(with_shared - without, _torch_ffn(L["x"], L["ws1"], L["ws2"]),
                               rtol=1e-10, atol=1e-12)


def check_layer_k_equals_E_is_full_mixture():
    """k = E: out = sum_e softmax_e * FFN_e(x) (scipy softmax, torch FFN)."""
    L = _small_layer(E=4)
    r = O.layer(L, 4)
    sm = scipy.special.softmax(L["x"].astype(np.float64) @ L["wg"].astype(np.float64).T, axis=1)
    want = sum(sm[:, e:e + 1] * _torch_ffn(L["x"], L["w1"][e], L["w2"][e]) for e in range(4))
    np.testing.assert_allclose(r["out"], want, rtol=1e-6, atol=1e-6)


def check_layer_rows_and_dispatched_form_agree():
    """The sampled-row evaluation and the dispatched buffer form equal the full layer."""
    L = _small_layer(E=4, Fs=16)
    r = O.layer(L, 2)
    toks = np.array([0, 5, 23])
    out_rows, _, _ = O.layer_rows(L, r["idx"], r["w"], toks)
    np.testing.assert_allclose(out_rows, r["out"][toks], rtol=1e-13, atol=1e-14)
    # expert-contiguous buffer: run each segment, gather back through inv
    ys = np.zeros((r["xs"].shape[0], L["x"].shape[1]))
    for e in range(4):
        a, b = r["offsets"][e], r["offsets"][e + 1]
        if b > a:
            ys[a:b] = O.expert_ffn(r["xs"][a:b], L["w1"][e], L["w2"][e])
    T, k = r["idx"].shape
    y = ys[r["inv"]].reshape(T, k, -1)
    np.testing.assert_allclose(O.combine(y, r["w"], r["ysh"]), r["out"], rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ stats

def check_capacity_closed_forms():
    want = {"tiny_fp32": 20, "mixtral_8x7b": 1280, "fine_grained_zipf": 320, "heavy_skew": 640}
    for name, cap in want.items():
        c = CONFIGS[name]
        counts = np.zeros(c.E, dtype=np.int64)
        counts[0] = c.T * c.k
        assert O.load_stats(counts, c.T, c.k, c.cf)["capacity"] == cap, name
    for T, cap in zip(DECODE_TOKENS, [0, 1, 2, 5, 10]):
        c = get_config(f"decode@T{T}")
        counts = np.zeros(c.E, dtype=np.int64)
        counts[0] = T * c.k
        assert O.load_stats(counts, T, c.k, c.cf)["capacity"] == cap, T


def check_stats_hand_fixture():
    cases = json.load(open(os.path.join(GOLDEN, "dispatch_stats_hand.json")))["cases"]
    for c in cases:
        st = O.load_stats(np.array(c["counts"]), c["T"], c["k"], c["cf"])
        for key in ["capacity", "overflow", "dropped", "drop_rate", "max_load", "min_load",
                    "gini_num", "gini_den", "gini", "straggler_ids"]:
            assert st[key] == c[key], (key, st[key], c[key])


def _gini_pairwise(c):
    n, tot = len(c), sum(c)
    if tot == 0:
        return Fraction(0)
    return Fraction(sum(abs(a - b) for a in c for b in c), 2 * n * tot)


def check_gini_closed_forms_and_brute_force():
    for n in [1, 2, 5, 8, 128, 256]:
        assert O.load_stats(np.full(n, 3), 3, 1, 1.0)["gini"] == 0.0
        one = np.zeros(n, dtype=np.int64); one[n // 2] = 7
        assert O.load_stats(one, 7, 1, 1.0)["gini"] == (n - 1) / n
    for n, m in [(128, 8), (256, 8), (10, 3)]:
        c = np.zeros(n, dtype=np.int64); c[:m] = 1
        assert O.load_stats(c, m, 1, 1.0)["gini"] == (n - m) / n
    # an all-zero count vector (only the Gini guard is under test here)
    assert O.load_stats(np.zeros(4, dtype=np.int64), 1, 1, 1.0)["gini"] == 0.0
    for n in range(1, 6):
        for c in itertools.product(range(5), repeat=n):
            st = O.load_stats(np.array(c), 1, 1, 1.0)
            g = _gini_pairwise(list(c))
            assert Fraction(st["gini_num"], st["gini_den"]) == g, c
            assert st["gini"] == float(g)
            assert abs(O.gini_page_formula(c) - float(g)) <= 8 * np.finfo(float).eps


def check_stats_single_decode_token():
    """T = 1, E = 128, k = 8: capacity 0, all 8 hits drop, skew = 1/(0 + 1e-5),
    Gini = (128 - 8)/128 = 0.9375, stragglers = the chosen ids ascending."""
    chosen = [100, 3, 77, 8, 120, 64, 0, 51]
    c = np.zeros(128, dtype=np.int64); c[chosen] = 1
    st = O.load_stats(c, 1, 8, 1.25)
    assert st["capacity"] == 0 and st["dropped"] == 8 and st["drop_rate"] == 1.0
    assert st["load_skew_ratio"] == 1.0 / (0.0 + 1e-5)
    assert st["gini"] == 0.9375
    assert st["straggler_ids"] == sorted(chosen) and st["num_stragglers"] == 8


def check_stats_strict_straggler_and_overflow():
    c = np.array([10, 11, 9, 30, 0])      # T*k = 60, E = 5, cf = 1 -> cap 12
    st = O.load_stats(c, 30, 2, 1.0)
    assert st["capacity"] == 12
    assert st["overflow"] == [0, 0, 0, 18, 0] and st["dropped"] == 18
    assert st["straggler_ids"] == [3]
    c = np.array([12, 12, 12, 12, 12])
    assert O.load_stats(c, 30, 2, 1.0)["straggler_ids"] == []


# ------------------------------------------------------------------ capacity-enforced dispatch

def check_dispatch_capped_hand_fixture():
    cases = json.load(open(os.path.join(GOLDEN, "dispatch_capped_hand.json")))["cases"]
    for c in cases:
        if "cf" in c:
            assert O.capacity(c["T"], c["k"], c["E"], c["cf"]) == c["cap"]
        x = np.arange(c["T"], dtype=np.float64)[:, None] * np.ones((1, 3))
        counts, offsets, perm, inv, xs = O.dispatch_capped(np.array(c["idx"]), x, c["E"], c["cap"])
        assert counts.tolist() == c["counts"]
        assert offsets.tolist() == c["offsets"]
        assert perm.tolist() == c["perm"]
        assert inv.tolist() == c["inv"]
        assert xs[:, 0].astype(int).tolist() == c["xs_tokens"]


def check_dispatch_capped_limits_and_prefix():
    """cap >= max count: the plain dispatch; cap = 0: nothing kept; otherwise each
    segment is the first cap rows of the plain segment, the dropped count is the
    statistics' overflow sum, and the kept rows are min(c, cap) per expert."""
    T, E, k = 97, 7, 3
    idx = _random_topk(T, E, k, 31)
    x = _rng(32).standard_normal((T, 5))
    full = O.dispatch(idx, x, E)
    big = O.dispatch_capped(idx, x, E, int(full[0].max()))
    for a, b in zip(full, big):
        assert np.array_equal(a, b)
    c0 = O.dispatch_capped(idx, x, E, 0)
    assert c0[1].tolist() == [0] * (E + 1) and c0[2].size == 0 and (c0[3] == -1).all()
    for cap in [1, 5, 40, 41, 50]:
        counts, offsets, perm, inv, xs = O.dispatch_capped(idx, x, E, cap)
        assert np.array_equal(counts, full[0])
        assert np.array_equal(np.diff(offsets), np.minimum(full[0], cap))
        for e in range(E):
            seg = perm[offsets[e]:offsets[e + 1]]
            assert np.array_equal(seg, full[2][full[1][e]:full[1][e] + seg.size])
        kept = inv >= 0
        assert np.array_equal(perm[inv[kept]], np.nonzero(kept)[0])
        cf = cap / (T * k / E)
        st = O.load_stats(counts, T, k, cf)
        if st["capacity"] == cap:
            assert int((~kept).sum()) == st["dropped"]
        assert np.array_equal(xs, x[perm // k])


def check_layer_capped_drops_terms():
    """A dropped assignment removes exactly its weighted expert output (no
    renormalisation); dropping everything leaves the shared expert only."""
    L = _small_layer(T=24, H=16, E=4, F=32, Fs=8)
    k = 2
    idx, w, _, _ = O.route(L["x"], L["wg"], L["bias"], k)
    tokens = np.arange(24)
    out_all, y, ysh = O.layer_rows(L, idx, w, tokens)
    keep = np.ones((24, k), dtype=bool)
    keep[3, 1] = False
    keep[10, 0] = False
    out_c, _, _ = O.layer_rows(L, idx, w, tokens, keep=keep)
    want = out_all.copy()
    want[3] -= float(w[3, 1]) * y[3, 1]
    want[10] -= float(w[10, 0]) * y[10, 0]
    np.testing.assert_allclose(out_c, want, rtol=0, atol=1e-12)
    out_none, _, _ = O.layer_rows(L, idx, w, tokens, keep=np.zeros((24, k), dtype=bool))
    np.testing.assert_allclose(out_none, ysh, rtol=0, atol=1e-15)


# ------------------------------------------------------------------ dynamic bias, aux statistics

def check_bias_update_closed_forms():
    """Loads above the mean lose gamma, below the mean gain gamma, at the mean keep B."""
    b = np.array([1.0, 2.0, 3.0, 4.0], dtype=np.float32)
    got = O.bias_update(b, [3, 1, 2, 2], 0.5)        # mean 2
    assert got.dtype == np.float32 and got.tolist() == [0.5, 2.5, 3.0, 4.0]
    got = O.bias_update(b, [8, 0, 0, 0], 0.25)       # one hot expert
    assert got.tolist() == [0.75, 2.25, 3.25, 4.25]
    assert O.bias_update(b, [5, 5, 5, 5], 0.5).tolist() == b.tolist()   # balanced
    assert O.bias_update(b, [0, 0, 0, 0], 0.5).tolist() == b.tolist()   # nothing routed
    # mean 7/3 is not an integer: 2 < 7/3 < 3
    assert O.bias_update(np.zeros(3, np.float32), [2, 3, 2], 1.0).tolist() == [1.0, -1.0, 1.0]


def check_bias_update_float32_rounding():
    """The result is B -/+ gamma rounded once to float32: 1 + 2^-25 rounds back to 1,
    and 2^24 + 1 is not representable either."""
    b = np.array([1.0, 16777216.0], dtype=np.float32)
    got = O.bias_update(b, [0, 4], 2.0 ** -25)
    assert got.tolist() == [1.0, 16777216.0]
    got = O.bias_update(b, [0, 4], 2.0 ** -23)
    assert got.tolist() == [1.0 + 2.0 ** -23, 16777216.0]


def check_bias_update_balances_a_constant_batch():
    """Scores equal to the bias alone (x = 0): every token picks the same top-k,
    so the chosen experts are overloaded and the rest idle; repeated updates
    must rotate the choice until every expert has been chosen (the rule's purpose)."""
    E, k, T, H = 6, 2, 12, 4
    bias = np.array([0.6, 0.5, 0.4, 0.3, 0.2, 0.1], dtype=np.float32)
    x = np.zeros((T, H))
    wg = np.zeros((E, H))
    seen = set()
    for _ in range(20):
        idx, _, _, _ = O.route(x, wg, bias, k)
        c = np.bincount(idx.ravel(), minlength=E)
        seen.update(idx[0].tolist())
        new = O.bias_update(bias, c, 0.25)
        hot = c > T * k / E
        assert (new[hot] < bias[hot]).all() and (new[~hot] > bias[~hot]).all()
        bias = new
    assert seen == set(range(E))


def check_load_fraction_closed_forms():
    """f_i = c_i / sum c: sums to 1; one step's counts give c_i / (T*k)."""
    assert O.load_fraction([3, 1, 2, 2]).tolist() == [0.375, 0.125, 0.25, 0.25]
    assert O.load_fraction([0, 0, 0]).tolist() == [0.0, 0.0, 0.0]
    T, E, k = 40, 8, 3
    idx = np.stack([_rng(40, t).permutation(E)[:k] for t in range(T)])
    c = np.bincount(idx.ravel(), minlength=E)
    f = O.load_fraction(c)
    assert int(c.sum()) == T * k
    for fe, ce in zip(f.tolist(), c.tolist()):      # each is c_i/(T*k) rounded once
        assert fe == float(Fraction(int(ce), T * k))
    assert abs(f.sum() - 1.0) <= 8 * np.finfo(float).eps


def check_prob_mean_closed_form():
    """Token 0 has scores ln(1..4) so p = (0.1, 0.2, 0.3, 0.4); token 1 has equal
    scores so p = 1/4 each. P = their average."""
    E, H = 4, 8
    wg = np.zeros((E, H))
    wg[:, 0] = np.log(np.arange(1, E + 1))
    x = np.zeros((2, H))
    x[0, 0] = 1.0
    _, _, _, p = O.route(x, wg, None, 2)
    np.testing.assert_allclose(O.prob_mean(p), [0.175, 0.225, 0.275, 0.325], rtol=0, atol=1e-15)
    # the same with the scores carried by the bias (B inside the softmax)
    _, _, _, p = O.route(np.zeros((3, H)), wg, np.log(np.arange(1, E + 1)).astype(np.float32), 1)
    np.testing.assert_allclose(O.prob_mean(p), [0.1, 0.2, 0.3, 0.4], rtol=1e-7)


def check_prob_mean_k_equals_E_matches_weights():
    """k = E: the renormalised weights are the softmax itself, so P_i is the mean
    weight the router gave expert i (scipy softmax gives the same)."""
    T, E, H = 30, 5, 16
    x = _rng(41).standard_normal((T, H))
    wg = _rng(42).standard_normal((E, H))
    b = _rng(43).standard_normal(E).astype(np.float32)
    idx, w, s, p = O.route(x, wg, b, E)
    P = O.prob_mean(p)
    Pw = np.zeros(E)
    for t in range(T):
        for j in range(E):
            Pw[idx[t, j]] += float(w[t, j]) / T
    np.testing.assert_allclose(P, Pw, atol=1e-7)
    np.testing.assert_allclose(P, scipy.special.softmax(x @ wg.T + b, axis=1).mean(0), atol=1e-12)
    assert abs(P.sum() - 1.0) < 1e-12


# ------------------------------------------------------------------ inputs

def check_widen_bf16_bit_patterns():
    """bf16 inputs are uint16 bit patterns (sign, 8 exponent bits, 7 fraction
    bits: the top half of an IEEE binary32); widen() must give their exact value.
    Hand-decoded patterns, then all 65536 patterns against torch's own
    bfloat16 -> float32 conversion (NaNs compared as NaNs)."""
    hand = {
        0x0000: 0.0, 0x3F80: 1.0, 0xBF80: -1.0, 0xC000: -2.0, 0x4040: 3.0,
        0x3F81: 1.0 + 2.0 ** -7,                    # one unit in the last place above 1
        0x3E80: 0.25,
        0x0001: 2.0 ** -133,                        # smallest subnormal: 2^-126 * 2^-7
        0x0080: 2.0 ** -126,                        # smallest normal
        0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127,     # largest finite
        0x7F80: math.inf, 0xFF80: -math.inf,
    }
    bits = np.array(list(hand), dtype=np.uint16)
    got = O.widen(bits)
    assert got.dtype == np.float64
    for b, v in zip(hand, got):
        assert v == hand[b], (hex(b), v, hand[b])
    neg0 = O.widen(np.array([0x8000], dtype=np.uint16))[0]
    assert neg0 == 0.0 and math.copysign(1.0, neg0) < 0
    with np.errstate(invalid="ignore"):   # signalling NaN patterns
        assert np.isnan(O.widen(np.array([0x7FC0, 0xFFC1], dtype=np.uint16))).all()
        every = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
        ref = torch.from_numpy(every.view(np.int16)).view(torch.bfloat16).float().double().numpy()
        got = O.widen(every)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # float32 inputs pass through exactly
    f = _rng(7).standard_normal(64).astype(np.float32)
    assert np.array_equal(O.widen(f), f.astype(np.float64))


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_")]

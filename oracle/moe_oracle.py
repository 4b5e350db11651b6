"""Plain, slow CPU oracle of one fine-grained MoE FFN layer forward.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import or call this
module; only the test suite, the smoke check and the benchmark's CPU-baseline
leg do. It shares no code with the HIP library.

Everything is float64 numpy on the exact input values (bf16 bit patterns are
widened exactly). Library primitives used as steps: matrix product, erf,
exp, argmax, nonzero. No blocking, fusion or reordering beyond the
definitions cited below.

Sources (the three web pages this layer is built from):
  [K3]  "hncyxsy.com Kimi K3 fine-grained MoE" article: the router listing
        (FineGrainedMoERouter: bias-free gate Linear, softmax over experts,
        top-k, divide the k weights by their sum), the dispatch/expert/combine
        three-stage flow, the always-on shared expert, and the FFN cost
        equation Time_comp = 2*B*S*K*(2*H*D_ffn)/FLOPs.
  [DIAG] "Kimi K3 专家路由不均衡诊断" (bjdmk.com.cn): section 3 diagnostics
        listing (MoERouteDiagnostics: histogram with add.at, capacity
        int(T*k/E*cf), overflow max(0, c - cap), drop rate, Gini, max/min skew,
        stragglers c > cap); section 4.1, the statistics f_i (share of the
        tokens routed to expert i) and P_i (mean router probability) of the
        auxiliary balance term; section 4.2, the biased score
        Score_i = Softmax(Logits_i + B_i) and the rule that nudges B_i down for
        an overloaded expert and up for an idle one.
  [BLOG] "lpqz.cn MoE engineering blog": section 3.1, expert = two Linear
        layers with GeLU; the dispatcher groups tokens by expert id, runs each
        expert on its group and scatters results back to the original order.

Readings where the pages are silent or garbled:
  * the routing bias sits inside the softmax, so it moves both the selection
    and the weights ([DIAG] 4.2);
  * top-k ids are in descending score order; ties go to the lower expert id;
  * GeLU is the erf form 0.5*a*(1+erf(a/sqrt(2)));
  * no Linear biases anywhere; weights use the [out, in] layout;
  * capacity drops are counted by the statistics; the capacity-enforcing
    dispatch keeps each expert's first cap assignments in token order and the
    dropped ones add nothing (no renormalisation of the kept weights);
  * the shared expert has weight 1 and is added to every token;
  * the residual add that follows the combine is not part of the layer output;
  * the bias rule compares each expert's count with the mean count; the step
    gamma is a caller's parameter (the page gives no value); f_i divides by
    the total count, so the f_i sum to 1 like the P_i.

Parity pins: every function here is pinned in tests/test_oracle_pins.py
against closed forms, hand-worked fixtures, brute force or library special
cases. None is "parity unpinned".
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
from scipy.special import erf as _erf


# ---------------------------------------------------------------- inputs

def widen(a) -> np.ndarray | None:
    """Exact float64 value of an input tensor (bf16 bits as uint16, or float32)."""
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        a = (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float64)


# ---------------------------------------------------------------- step 1: route

def logits(x, wg, bias=None) -> np.ndarray:
    """Gate scores s[t, e] = sum_h x[t, h] * Wg[e, h] (+ B_e).

    [K3] router listing: a gate Linear with no bias, Wg in [E, H] layout;
    [DIAG] 4.2: the per-expert bias B is added to the logits.
    """
    s = widen(x) @ widen(wg).T
    if bias is not None:
        s = s + widen(bias)[None, :]
    return s


def route(x, wg, bias, k: int):
    """Top-k routing of every token.

    [K3] router listing: softmax over all experts, take the k largest
    probabilities in descending order, then divide them by their sum.
    [DIAG] 4.2: the softmax runs over Logits + B.
    Selection is k rounds of arg-max over the probabilities; arg-max returns
    the lowest id among equals (tie rule).

    Returns (idx int32 [T, k], w float32 [T, k], s float64 [T, E], p float64 [T, E]).
    """
    s = logits(x, wg, bias)
    T, E = s.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    m = s.max(axis=1, keepdims=True)
    z = np.exp(s - m)
    p = z / z.sum(axis=1, keepdims=True)           # softmax over all E experts
    idx = np.empty((T, k), dtype=np.int32)
    sel = np.empty((T, k), dtype=np.float64)
    remaining = p.copy()
    for j in range(k):
        best = np.argmax(remaining, axis=1)        # first (lowest id) maximum
        idx[:, j] = best
        sel[:, j] = p[np.arange(T), best]
        remaining[np.arange(T), best] = -np.inf
    w = sel / sel.sum(axis=1, keepdims=True)       # renormalise the k weights
    return idx, w.astype(np.float32), s, p


# ---------------------------------------------------------------- step 2: dispatch

def dispatch(idx, x, E: int):
    """Group the (token, slot) assignments by expert.

    [DIAG] section 3: per-expert hit counts by add.at over the flattened ids.
    [BLOG] section 3.1 dispatcher: for each expert id in turn, mask the ids
    equal to it and take the positions where the mask holds; the gathered rows
    of all experts sit in one shared buffer, expert after expert.
    Assignment a = t*k + j. perm[p] = a for buffer row p; inv[a] = p;
    xs[p] = x[perm[p] // k] (exact copy).
    """
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    flat = idx.reshape(-1)
    counts = np.zeros(E, dtype=np.int64)
    np.add.at(counts, flat, 1)
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    perm = np.empty(T * k, dtype=np.int64)
    inv = np.empty(T * k, dtype=np.int64)
    for e in range(E):
        where = np.nonzero(flat == e)[0]            # ascending assignment order
        start = offsets[e]
        perm[start:start + where.size] = where
        inv[where] = np.arange(start, start + where.size)
    xs = np.asarray(x)[perm // k]
    return (counts.astype(np.int32), offsets.astype(np.int32), perm.astype(np.int32),
            inv.astype(np.int32), xs)


def capacity(T: int, k: int, E: int, cf: float) -> int:
    """int((T*k/E) * cf) in float64, in that order ([DIAG] section 3 listing)."""
    return int(((T * k) / E) * cf)


def dispatch_capped(idx, x, E: int, cap: int):
    """Dispatch with the expert capacity enforced ([DIAG] section 3 counts the
    assignments beyond an expert's capacity as dropped; section 5 describes
    dropping them). Each expert keeps its first ``cap`` assignments in token
    order (the stable order of dispatch()); later ones are dropped: they get
    no buffer row and inv = -1. counts are the raw counts (before dropping);
    offsets are those of the kept rows. Returns (counts, offsets, perm, inv, xs)
    with perm and xs holding the kept rows only."""
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    flat = idx.reshape(-1)
    counts = np.zeros(E, dtype=np.int64)
    np.add.at(counts, flat, 1)
    kept = np.minimum(counts, cap)
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + kept[e]
    perm = np.empty(offsets[E], dtype=np.int64)
    inv = np.full(T * k, -1, dtype=np.int64)
    for e in range(E):
        where = np.nonzero(flat == e)[0][:cap]     # the first cap, ascending assignment order
        start = offsets[e]
        perm[start:start + where.size] = where
        inv[where] = np.arange(start, start + where.size)
    xs = np.asarray(x)[perm // k]
    return (counts.astype(np.int32), offsets.astype(np.int32), perm.astype(np.int32),
            inv.astype(np.int32), xs)


def kept_mask(inv) -> np.ndarray:
    """True for assignments that kept a buffer row (inv >= 0)."""
    return np.asarray(inv) >= 0


# ---------------------------------------------------------------- step 3: experts

def gelu_erf(a: np.ndarray) -> np.ndarray:
    """GeLU, erf form: 0.5 * a * (1 + erf(a / sqrt(2)))."""
    return 0.5 * a * (1.0 + _erf(a / math.sqrt(2.0)))


def expert_ffn(rows, w1, w2) -> np.ndarray:
    """One expert on a block of rows: Linear -> GeLU -> Linear, no biases.

    [BLOG] section 3.1: each expert is two Linear layers with a GeLU between.
    W1 [F, H] and W2 [H, F] in the [out, in] layout; rows [n, H].
    """
    a = widen(rows) @ widen(w1).T
    return gelu_erf(a) @ widen(w2).T


def expert_outputs(x, idx, w1, w2, tokens=None) -> np.ndarray:
    """y[t, j] = FFN_{idx[t, j]}(x[t]) for the given tokens (all by default).

    The direct definition: every token meets each of its chosen experts. Rows
    that choose the same expert are evaluated together in one product.
    Returns float64 [n_tokens, k, H].
    """
    idx = np.asarray(idx)
    if tokens is None:
        tokens = np.arange(idx.shape[0])
    tokens = np.asarray(tokens)
    sub = idx[tokens]
    n, k = sub.shape
    H = np.asarray(x).shape[1]
    y = np.zeros((n, k, H), dtype=np.float64)
    for e in np.unique(sub):
        r, j = np.nonzero(sub == e)
        y[r, j] = expert_ffn(np.asarray(x)[tokens[r]], w1[e], w2[e])
    return y


def shared_outputs(x, ws1, ws2, tokens=None) -> np.ndarray | None:
    """The always-on shared expert, weight 1 ([K3] introduction)."""
    if ws1 is None:
        return None
    xs = np.asarray(x) if tokens is None else np.asarray(x)[np.asarray(tokens)]
    return expert_ffn(xs, ws1, ws2)


# ---------------------------------------------------------------- step 4: combine

def combine(y, w, ysh=None) -> np.ndarray:
    """out[t] = sum_j w[t, j] * y[t, j] (j ascending) + ysh[t].

    [K3] combine phase: expert outputs are weighted and summed back at the
    token's owner. y is [T, k, H] (per assignment, token order).
    """
    w = np.asarray(w, dtype=np.float64)
    out = np.zeros((y.shape[0], y.shape[2]), dtype=np.float64)
    for j in range(y.shape[1]):
        out += w[:, j:j + 1] * y[:, j]
    if ysh is not None:
        out += ysh
    return out


def layer(L: dict, k: int):
    """The whole layer on every token: returns a dict of all step results."""
    idx, w, s, p = route(L["x"], L["wg"], L["bias"], k)
    E = np.asarray(L["wg"]).shape[0]
    counts, offsets, perm, inv, xs = dispatch(idx, L["x"], E)
    y = expert_outputs(L["x"], idx, L["w1"], L["w2"])
    ysh = shared_outputs(L["x"], L["ws1"], L["ws2"])
    out = combine(y, w, ysh)
    return dict(idx=idx, w=w, s=s, p=p, counts=counts, offsets=offsets, perm=perm, inv=inv,
                xs=xs, y=y, ysh=ysh, out=out)


def layer_rows(L: dict, idx, w, tokens, keep=None):
    """Layer output for a sample of tokens, given their routing (idx, w).

    keep (optional bool [T, k]): assignments that were not dropped; a dropped
    assignment adds nothing and the kept weights are not renormalised."""
    tokens = np.asarray(tokens)
    y = expert_outputs(L["x"], idx, L["w1"], L["w2"], tokens)
    ysh = shared_outputs(L["x"], L["ws1"], L["ws2"], tokens)
    wt = np.asarray(w, dtype=np.float64)[tokens]
    if keep is not None:
        wt = np.where(np.asarray(keep)[tokens], wt, 0.0)
    return combine(y, wt, ysh), y, ysh


# ---------------------------------------------------------------- step 5: load stats

def load_stats(counts, T: int, k: int, cf: float) -> dict:
    """Per-step load diagnostics of [DIAG] section 3.

    capacity = int((T*k/E) * cf) evaluated in float64, in that order;
    overflow_e = max(0, c_e - capacity); dropped = sum overflow (counted only);
    drop_rate = dropped / (T*k); skew = max / (min + 1e-5);
    stragglers = ids with c_e > capacity, ascending.
    Gini: 0 when the counts sum to 0; otherwise the page's sorted-index form
    2*sum(i*c_(i))/(n*sum c) - (n+1)/n with c sorted ascending and i = 1..n,
    kept as the exact fraction (2*sum(i*c_(i)) - (n+1)*sum c) / (n*sum c) and
    rounded to float64 by one division.
    """
    c = [int(v) for v in np.asarray(counts).tolist()]
    E = len(c)
    assignments = T * k
    capacity = int((assignments / E) * cf)
    overflow = [max(0, v - capacity) for v in c]
    dropped = sum(overflow)
    total = sum(c)
    if total == 0:
        gini_num, gini_den, gini = 0, 1, 0.0
    else:
        srt = sorted(c)
        gini_num = 2 * sum((i + 1) * v for i, v in enumerate(srt)) - (E + 1) * total
        gini_den = E * total
        gini = gini_num / gini_den          # Python int / int: correctly rounded
    mx, mn = max(c), min(c)
    stragglers = [e for e in range(E) if c[e] > capacity]
    return dict(num_tokens=T, assignments=assignments, capacity=capacity, max_load=mx,
                min_load=mn, dropped=dropped, num_stragglers=len(stragglers),
                gini_num=gini_num, gini_den=gini_den,
                load_skew_ratio=float(mx) / (float(mn) + 1e-5), gini=gini,
                drop_rate=float(dropped) / float(assignments),
                overflow=overflow, straggler_ids=stragglers)


# ---------------------------------------------------------------- next: dynamic bias, aux statistics

def load_fraction(counts) -> np.ndarray:
    """f_i = c_i / sum_e c_e, the share of the routed assignments that expert i
    received ([DIAG] section 4.1, the f_i of the auxiliary balance term). With
    one step's counts the denominator is T*k. All zeros when nothing was routed.
    Returns float64 [E]."""
    c = np.asarray(counts, dtype=np.int64)
    total = int(c.sum())
    if total == 0:
        return np.zeros(c.size, dtype=np.float64)
    return c.astype(np.float64) / float(total)


def prob_mean(p) -> np.ndarray:
    """P_i = mean over the T tokens of the router probability p[t, i]
    ([DIAG] section 4.1, the P_i of the auxiliary balance term). p is the full
    softmax over all E experts that route() returns, i.e. of Logits + B.
    Returns float64 [E]."""
    p = np.asarray(p, dtype=np.float64)
    return p.sum(axis=0) / p.shape[0]


def bias_update(bias, counts, gamma):
    """One step of the dynamic routing-bias rule ([DIAG] section 4.2).

    An expert whose load is above the mean load sum(c)/E is overloaded: its
    bias drops by gamma. One below the mean is idle: its bias rises by gamma.
    One exactly at the mean keeps its bias. The counts may be one step's or
    summed over a window of steps; the rule only compares each count with
    their mean (exactly, in integers). Computed in float64 on the float32
    inputs, rounded once to float32. Returns float32 [E].
    """
    b = widen(np.asarray(bias, dtype=np.float32))
    g = float(np.float32(gamma))
    c = [int(v) for v in np.asarray(counts).tolist()]
    E = len(c)
    mean = Fraction(sum(c), E)
    out = np.empty(E, dtype=np.float64)
    for e in range(E):
        if c[e] > mean:
            out[e] = b[e] - g
        elif c[e] < mean:
            out[e] = b[e] + g
        else:
            out[e] = b[e]
    return out.astype(np.float32)


def gini_page_formula(counts) -> float:
    """The page's floating-point Gini expression, for cross-checking the exact form."""
    c = np.sort(np.asarray(counts, dtype=np.float64))
    n = c.size
    if c.sum() == 0:
        return 0.0
    i = np.arange(1, n + 1)
    return float((2 * np.sum(i * c)) / (n * np.sum(c)) - (n + 1) / n)

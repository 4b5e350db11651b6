"""Plant plausible mistakes in the oracle (CPU only) and require a pin to catch each.

A pin set that lets a dropped term, a wrong sign, a wrong index or a swapped
operand through is not a pin; these tests show the checks in tests/pins.py
are sensitive to each such mistake.
"""
import math

import numpy as np
import pytest

import oracle.moe_oracle as O
from tests import pins

_route, _combine, _load_stats, _dispatch, _ffn = O.route, O.combine, O.load_stats, O.dispatch, O.expert_ffn


def m_no_renormalise(mp):
    def route(x, wg, b, k):
        idx, w, s, p = _route(x, wg, b, k)
        return idx, np.take_along_axis(p, idx.astype(np.int64), 1).astype(np.float32), s, p
    mp.setattr(O, "route", route)


def m_select_smallest(mp):
    def route(x, wg, b, k):
        _, _, s, p = _route(x, wg, b, k)
        idx = np.argsort(s, axis=1, kind="stable")[:, :k].astype(np.int32)
        sel = np.take_along_axis(p, idx.astype(np.int64), 1)
        return idx, (sel / sel.sum(1, keepdims=True)).astype(np.float32), s, p
    mp.setattr(O, "route", route)


def m_bias_selection_only(mp):
    def route(x, wg, b, k):
        idx, _, s, p = _route(x, wg, b, k)
        s0 = O.widen(x) @ O.widen(wg).T
        z = np.exp(s0 - s0.max(1, keepdims=True))
        sel = np.take_along_axis(z, idx.astype(np.int64), 1)
        return idx, (sel / sel.sum(1, keepdims=True)).astype(np.float32), s, p
    mp.setattr(O, "route", route)


def m_ties_to_higher_id(mp):
    def route(x, wg, b, k):
        E = np.asarray(wg).shape[0]
        idx, w, s, p = _route(x, np.asarray(wg)[::-1], None if b is None else np.asarray(b)[::-1], k)
        return (E - 1 - idx).astype(np.int32), w, s[:, ::-1], p[:, ::-1]
    mp.setattr(O, "route", route)


def m_unstable_dispatch(mp):
    def dispatch(idx, x, E):
        counts, offsets, perm, inv, xs = _dispatch(idx, x, E)
        k = np.asarray(idx).shape[1]
        for e in range(E):
            a, b = offsets[e], offsets[e + 1]
            perm[a:b] = perm[a:b][::-1].copy()
        inv[perm] = np.arange(perm.size)
        return counts, offsets, perm, inv, np.asarray(x)[perm // k]
    mp.setattr(O, "dispatch", dispatch)


def m_offsets_inclusive(mp):
    def dispatch(idx, x, E):
        counts, offsets, perm, inv, xs = _dispatch(idx, x, E)
        return counts, np.concatenate([offsets[1:], offsets[-1:]]), perm, inv, xs
    mp.setattr(O, "dispatch", dispatch)


def m_gelu_tanh(mp):
    mp.setattr(O, "gelu_erf", lambda a: 0.5 * a * (1 + np.tanh(math.sqrt(2 / math.pi) * (a + 0.044715 * a ** 3))))


def m_gelu_dropped(mp):
    mp.setattr(O, "gelu_erf", lambda a: a)


def m_gelu_sign(mp):
    mp.setattr(O, "gelu_erf", lambda a: 0.5 * a * (1 - O._erf(a / math.sqrt(2))))


def m_w2_layout_misread(mp):
    """W2 stored [H, F] but read as if it were [F, H] (a swapped-layout mistake)."""
    def expert_ffn(rows, w1, w2):
        g = O.gelu_erf(O.widen(rows) @ O.widen(w1).T)
        w2 = O.widen(w2)
        return g @ w2.reshape(w2.shape[1], w2.shape[0])
    mp.setattr(O, "expert_ffn", expert_ffn)


def m_w1_layout_misread(mp):
    """W1 stored [F, H] but read as if it were [H, F]."""
    def expert_ffn(rows, w1, w2):
        w1 = O.widen(w1)
        g = O.gelu_erf(O.widen(rows) @ w1.reshape(w1.shape[1], w1.shape[0]))
        return g @ O.widen(w2).T
    mp.setattr(O, "expert_ffn", expert_ffn)


def m_combine_drops_shared(mp):
    mp.setattr(O, "combine", lambda y, w, ysh=None: _combine(y, w, None))


def m_combine_weights_swapped(mp):
    mp.setattr(O, "combine", lambda y, w, ysh=None: _combine(y, np.asarray(w)[:, ::-1], ysh))


def m_capacity_ceil(mp):
    def load_stats(counts, T, k, cf):
        st = _load_stats(counts, T, k, cf)
        cap = math.ceil((T * k / len(counts)) * cf)
        c = [int(v) for v in counts]
        st.update(capacity=cap, overflow=[max(0, v - cap) for v in c],
                  straggler_ids=[e for e, v in enumerate(c) if v > cap])
        st["dropped"] = sum(st["overflow"])
        return st
    mp.setattr(O, "load_stats", load_stats)


def m_gini_index_from_zero(mp):
    def load_stats(counts, T, k, cf):
        st = _load_stats(counts, T, k, cf)
        c = sorted(int(v) for v in counts)
        n, tot = len(c), sum(c)
        if tot:
            st["gini_num"] = 2 * sum(i * v for i, v in enumerate(c)) - (n + 1) * tot
            st["gini"] = st["gini_num"] / st["gini_den"]
        return st
    mp.setattr(O, "load_stats", load_stats)


def m_straggler_ge(mp):
    def load_stats(counts, T, k, cf):
        st = _load_stats(counts, T, k, cf)
        st["straggler_ids"] = [e for e, v in enumerate(counts) if int(v) >= st["capacity"]]
        return st
    mp.setattr(O, "load_stats", load_stats)


_bias_update, _load_fraction, _prob_mean = O.bias_update, O.load_fraction, O.prob_mean


def m_bias_update_sign_flipped(mp):
    mp.setattr(O, "bias_update", lambda b, c, g: _bias_update(b, c, -g))


def m_bias_update_mean_floor(mp):
    """Compare with the mean rounded down (integer division) instead of the exact mean."""
    def bias_update(b, c, g):
        c = [int(v) for v in c]
        m = sum(c) // len(c)
        b = np.asarray(b, dtype=np.float64)
        return np.array([b[e] - g if c[e] > m else b[e] + g if c[e] < m else b[e]
                         for e in range(len(c))], dtype=np.float32)
    mp.setattr(O, "bias_update", bias_update)


def m_bias_update_in_float64(mp):
    """Result left in float64 (no rounding to the float32 bias)."""
    def bias_update(b, c, g):
        c = [int(v) for v in c]
        b = np.asarray(b, dtype=np.float64)
        E = len(c)
        return np.array([b[e] - g if c[e] * E > sum(c) else b[e] + g if c[e] * E < sum(c) else b[e]
                         for e in range(E)])
    mp.setattr(O, "bias_update", bias_update)


def m_load_fraction_per_token(mp):
    """f_i = c_i / T (tokens) instead of c_i / (T*k) (assignments)."""
    def load_fraction(c):
        c = np.asarray(c, dtype=np.int64)
        return _load_fraction(c) * 2 if c.sum() else _load_fraction(c)
    mp.setattr(O, "load_fraction", load_fraction)


def m_prob_mean_is_sum(mp):
    mp.setattr(O, "prob_mean", lambda p: np.asarray(p).sum(axis=0))


def m_prob_mean_first_token(mp):
    mp.setattr(O, "prob_mean", lambda p: np.asarray(p, dtype=np.float64)[0].copy())


_dispatch_capped, _layer_rows = O.dispatch_capped, O.layer_rows


def m_capped_keeps_last(mp):
    """Keep the last cap assignments of each expert instead of the first."""
    def dispatch_capped(idx, x, E, cap):
        idx = np.asarray(idx)
        T, k = idx.shape
        rev = idx[::-1].copy()
        counts, offsets, perm, inv, _ = _dispatch_capped(rev, x[::-1] if x is not None else x, E, cap)
        a_rev = perm.astype(np.int64)
        t = T - 1 - a_rev // k
        perm2 = (t * k + a_rev % k).astype(np.int32)
        for e in range(E):
            a, b = offsets[e], offsets[e + 1]
            perm2[a:b] = np.sort(perm2[a:b])
        inv2 = np.full(T * k, -1, dtype=np.int32)
        inv2[perm2] = np.arange(perm2.size)
        return counts, offsets, perm2, inv2, np.asarray(x)[perm2 // k]
    mp.setattr(O, "dispatch_capped", dispatch_capped)


def m_capped_off_by_one(mp):
    mp.setattr(O, "dispatch_capped", lambda idx, x, E, cap: _dispatch_capped(idx, x, E, cap + 1))


def m_capped_renormalises(mp):
    def layer_rows(L, idx, w, tokens, keep=None):
        if keep is None:
            return _layer_rows(L, idx, w, tokens)
        wk = np.where(keep, np.asarray(w, dtype=np.float64), 0.0)
        s = wk.sum(axis=1, keepdims=True)
        wk = np.where(s > 0, wk / np.where(s > 0, s, 1.0), 0.0)
        return _layer_rows(L, idx, wk, tokens, keep=keep)
    mp.setattr(O, "layer_rows", layer_rows)


_widen = O.widen


def m_widen_as_float16(mp):
    """Read the 16-bit patterns as IEEE half precision instead of bf16."""
    def widen(a):
        a = None if a is None else np.asarray(a)
        if a is not None and a.dtype == np.uint16:
            return a.view(np.float16).astype(np.float64)
        return _widen(a)
    mp.setattr(O, "widen", widen)


def m_widen_shift_15(mp):
    """Shift the bf16 bits into the float32 word one place short."""
    def widen(a):
        a = None if a is None else np.asarray(a)
        if a is not None and a.dtype == np.uint16:
            return (a.astype(np.uint32) << 15).view(np.float32).astype(np.float64)
        return _widen(a)
    mp.setattr(O, "widen", widen)


MUTATIONS = [m_widen_as_float16, m_widen_shift_15, m_no_renormalise, m_select_smallest, m_bias_selection_only, m_ties_to_higher_id,
             m_unstable_dispatch, m_offsets_inclusive, m_gelu_tanh, m_gelu_dropped, m_gelu_sign,
             m_w2_layout_misread, m_w1_layout_misread, m_combine_drops_shared, m_combine_weights_swapped, m_capacity_ceil,
             m_gini_index_from_zero, m_straggler_ge, m_bias_update_sign_flipped,
             m_bias_update_mean_floor, m_bias_update_in_float64, m_load_fraction_per_token,
             m_prob_mean_is_sum, m_prob_mean_first_token, m_capped_keeps_last,
             m_capped_off_by_one, m_capped_renormalises]


@pytest.mark.parametrize("mutate", MUTATIONS, ids=lambda f: f.__name__)
def test_planted_mistake_is_caught(mutate, monkeypatch):
    mutate(monkeypatch)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check()
        except Exception as exc:  # an assertion or a shape error both count
            caught.append((check.__name__, type(exc).__name__))
    assert caught, f"no pin caught {mutate.__name__}"

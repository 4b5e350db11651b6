"""CPU checks of the parity harness itself (no GPU).

The GPU tests compare the library's outputs with the oracle through
tests/parity.py. Here the "GPU result" is the oracle's own output rounded to
bf16, so the harness must accept it; then single planted faults (one wrong
row, one stale 32-row block, a dropped assignment that still contributes)
must be rejected, including ones the whole-tensor norm alone would let through.
"""
import numpy as np
import pytest

import oracle
from synth import MoEConfig, f32_to_bf16_bits
from tests.parity import TOL_BF16_REL_L2, check_values, token_chunk
from tests.support import conditioned_layer

CFG = MoEConfig("harness_bf16", T=300, H=128, E=8, k=2, F=128, Fs=64, bias_amp=1.0)


def _bf16(a):
    return f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def _oracle_as_gpu(cfg, L, keep_cap=None):
    T, k, E = cfg.T, cfg.k, cfg.E
    idx, w, _, _ = oracle.route(L["x"], L["wg"], L["bias"], k)
    if keep_cap is None:
        _, _, perm, inv, _ = oracle.dispatch(idx, np.empty((T, 0)), E)
        keep = None
    else:
        _, _, perm, inv, _ = oracle.dispatch_capped(idx, np.empty((T, 0)), E, keep_cap)
        keep = oracle.kept_mask(inv).reshape(T, k)
    out, y, ysh = oracle.layer_rows(L, idx, w, np.arange(T), keep=keep)
    ys = np.zeros((T * k, cfg.H), dtype=np.float64)
    kept = inv >= 0
    ys[inv[kept]] = y.reshape(T * k, -1)[kept]
    return idx, w, inv, keep, _bf16(out), _bf16(ys), _bf16(ysh)


def test_harness_accepts_the_rounded_oracle_and_rejects_planted_faults():
    cfg, L, _ = conditioned_layer(CFG)
    idx, w, inv, _, out, ys, ysh = _oracle_as_gpu(cfg, L)
    rep = check_values(cfg, L, idx, w, out, ys_got=ys, inv=inv, ysh_got=ysh)
    assert rep["out_rel_l2"] < 5e-3 and rep["out_rows"] == cfg.T
    assert rep["ys_rows"] == cfg.T * cfg.k and rep["ysh_rows"] == cfg.T

    # one token row scaled by 1.1: the whole-tensor norm stays far below the
    # bar, the per-row bound catches it
    bad = out.copy()
    bad[17] = _bf16(oracle.widen(out[17]) * 1.1)
    whole = np.linalg.norm(oracle.widen(bad) - oracle.widen(out)) / np.linalg.norm(oracle.widen(out))
    assert whole < TOL_BF16_REL_L2
    with pytest.raises(AssertionError, match="a row"):
        check_values(cfg, L, idx, w, bad, ys_got=ys, inv=inv, ysh_got=ysh)

    # a 32-row block of expert rows left stale (zeros): caught on ys
    stale = ys.copy()
    stale[64:96] = 0
    with pytest.raises(AssertionError, match="ys"):
        check_values(cfg, L, idx, w, out, ys_got=stale, inv=inv, ysh_got=ysh)

    # the shared rows of one token wrong
    bad_sh = ysh.copy()
    bad_sh[5] = _bf16(-oracle.widen(ysh[5]))
    with pytest.raises(AssertionError, match="ysh"):
        check_values(cfg, L, idx, w, out, ys_got=ys, inv=inv, ysh_got=bad_sh)


def test_harness_chunks_cover_every_token():
    cfg = MoEConfig("chunked", T=5000, H=4096, E=8, k=8, F=64)
    n = token_chunk(cfg)
    assert n == (1 << 27) // (8 * 4096) and n < cfg.T
    covered = np.concatenate([np.arange(a, min(cfg.T, a + n)) for a in range(0, cfg.T, n)])
    assert np.array_equal(covered, np.arange(cfg.T))


def test_harness_capped_layer_zero_rows():
    """Capacity 0 without a shared expert: every output row is zero and must
    come back as exactly zero; a row with any value is rejected."""
    cfg, L, _ = conditioned_layer(MoEConfig("harness_cap0", T=40, H=64, E=4, k=2, F=64))
    idx, w, inv, keep, out, ys, _ = _oracle_as_gpu(cfg, L, keep_cap=0)
    assert not keep.any() and (inv < 0).all()
    rep = check_values(cfg, L, idx, w, out, ys_got=ys, inv=inv, keep=keep)
    assert rep["out_rows"] == cfg.T and "ys_rows" not in rep
    bad = out.copy()
    bad[3, 7] = 0x3F80
    with pytest.raises(AssertionError, match="should be zero"):
        check_values(cfg, L, idx, w, bad, ys_got=ys, inv=inv, keep=keep)

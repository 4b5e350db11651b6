"""Graph replay of the five calls (decode latency), checked against the oracle.

Several replays with different inputs, with eager work and synchronisations in
between. Every replay is compared with the CPU oracle on the same inputs
(routing, dispatch and statistics bit for bit; the expert rows, shared rows
and output over every token, whole tensor and row by row) and with an eager
run of the same input bit for bit (same kernels, same order, no atomics).
Each replay's x is a fresh seeded draw held to the same gap rule as every
parity input, so the routing decision is unique.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_05_amd as moe
from sparse_mixture_experts_05_amd.binding import read_stats
from synth import MoEConfig, get_config, make_layer, redraw_rows
from tests.parity import (GAMMA, TOL_P, check_routing, check_stats, check_values, to_dev,
                          to_host)
from tests.support import condition_x

pytestmark = pytest.mark.gpu


# decode shapes (small-segment GEMM) and a skewed mid-size layer on the 256x256
# kernel with its planning launch, split over short segments in tile pairs
GRAPH_CASES = ["decode@T1", "decode@T16",
               MoEConfig("graph_big_pairs", T=1024, H=512, E=16, k=4, F=512, Fs=256, bias_amp=2.0)]


def _replay_input(cfg, L, rep, bias=None):
    """Layer dict for replay `rep`: x drawn from the stream [seed, 8, t, 100 + rep]
    and conditioned by the gap rule under `bias` (the layer's own if None)."""
    Lr = dict(L)
    if bias is not None:
        Lr["bias"] = bias
    Lr["x"] = redraw_rows(cfg, np.arange(cfg.T), 100 + rep)
    condition_x(cfg, Lr)
    return Lr


def _check_replay(cfg, Lr, g, keep_cap=None):
    """The graph's static outputs after a replay against the oracle on Lr."""
    T, k, E = cfg.T, cfg.k, cfg.E
    got = {"topk_idx": to_host(g.idx), "topk_w": to_host(g.w)}
    report = {}
    idx, w, p = check_routing(cfg, Lr, got, report)
    if keep_cap is None:
        counts, offsets, perm, inv, _ = oracle.dispatch(idx, np.empty((T, 0)), E)
        keep = None
    else:
        counts, offsets, perm, inv, _ = oracle.dispatch_capped(idx, np.empty((T, 0)), E, keep_cap)
        keep = oracle.kept_mask(inv).reshape(T, k)
    n = int(offsets[-1])
    assert np.array_equal(to_host(g.dsp["counts"]), counts)
    assert np.array_equal(to_host(g.dsp["offsets"]), offsets)
    assert np.array_equal(to_host(g.dsp["perm"])[:n], perm)
    assert np.array_equal(to_host(g.dsp["inv"]), inv)
    check_stats(cfg, counts, read_stats(g.stats, g.overflow, g.stragglers), report)
    check_values(cfg, Lr, idx, w, to_host(g.out), ys_got=to_host(g.ys), inv=inv, keep=keep,
                 ysh_got=to_host(g.ysh), report=report)
    return report, counts, p


@pytest.mark.parametrize("case", GRAPH_CASES, ids=lambda c: c if isinstance(c, str) else c.name)
def test_graph_replays_match_oracle_and_eager(case):
    cfg = get_config(case) if isinstance(case, str) else case
    L = make_layer(cfg)
    d = {k: to_dev(v) for k, v in L.items()}
    print(f"\n[gpu] graph {cfg.name}", flush=True)
    g = moe.MoELayerGraph(d["wg"], d["bias"], d["w1"], d["w2"], cfg.k, cfg.T, ws1=d["ws1"],
                          ws2=d["ws2"], capacity_factor=cfg.cf)
    for rep in range(4):
        Lr = _replay_input(cfg, L, rep)
        xr = to_dev(Lr["x"])
        out_g = to_host(g.run(xr).clone())
        torch.cuda.synchronize()
        report, _, _ = _check_replay(cfg, Lr, g)
        print(f"[gpu] graph {cfg.name} replay {rep}: {report}", flush=True)
        eager = moe.moe_layer_forward(xr, d["wg"], d["bias"], d["w1"], d["w2"], cfg.k,
                                      ws1=d["ws1"], ws2=d["ws2"])
        torch.cuda.synchronize()
        assert np.array_equal(to_host(g.idx), to_host(eager["topk_idx"])), rep
        assert np.array_equal(out_g, to_host(eager["out"])), rep


def test_graph_with_bias_feedback_matches_oracle_and_eager_loop():
    """The graph with the dynamic-bias step: each replay routes with the bias the
    previous replay wrote. After every replay the routing, output, mean
    probabilities, load fractions and the new bias match the oracle run with
    the bias the replay started from, and an eager loop on its own bias copy
    gives the same bits."""
    cfg = get_config("decode@T32")
    L = make_layer(cfg)
    d = {k: to_dev(v) for k, v in L.items()}
    E = cfg.E
    gamma = 0.05
    b_graph = torch.zeros(E, dtype=torch.float32, device="cuda")
    b_eager = torch.zeros(E, dtype=torch.float32, device="cuda")
    print("\n[gpu] graph with bias feedback decode@T32", flush=True)
    g = moe.MoELayerGraph(d["wg"], b_graph, d["w1"], d["w2"], cfg.k, cfg.T, ws1=d["ws1"],
                          ws2=d["ws2"], capacity_factor=cfg.cf, bias_gamma=gamma)
    assert (to_host(b_graph) == 0).all()          # warm-up did not move the bias
    pm = torch.empty(E, dtype=torch.float32, device="cuda")
    frac = torch.empty(E, dtype=torch.float32, device="cuda")
    moved = 0
    for rep in range(5):
        b_before = to_host(b_graph).copy()
        Lr = _replay_input(cfg, L, 200 + rep, bias=b_before)
        xr = to_dev(Lr["x"])
        out_g = to_host(g.run(xr).clone())
        torch.cuda.synchronize()
        report, counts, p = _check_replay(cfg, Lr, g)
        P = oracle.prob_mean(p)
        perr = float((np.abs(to_host(g.prob_mean).astype(np.float64) - P) / P).max())
        assert perr <= TOL_P, (rep, perr)
        b_ref = oracle.bias_update(b_before, counts, gamma)
        assert np.array_equal(to_host(b_graph).view(np.uint32), b_ref.view(np.uint32)), rep
        f_ref = oracle.load_fraction(counts).astype(np.float32)
        assert np.array_equal(to_host(g.load_frac).view(np.uint32), f_ref.view(np.uint32)), rep
        print(f"[gpu] bias feedback replay {rep}: {report}, prob_mean_max_rel={perr:.2e}",
              flush=True)
        r = moe.moe_layer_forward(xr, d["wg"], b_eager, d["w1"], d["w2"], cfg.k, ws1=d["ws1"],
                                  ws2=d["ws2"], prob_mean=pm)
        moe.moe_bias_update(r["counts"], b_eager, gamma, load_frac=frac)
        torch.cuda.synchronize()
        assert np.array_equal(out_g, to_host(r["out"])), rep
        assert np.array_equal(to_host(g.prob_mean), to_host(pm)), rep
        assert np.array_equal(to_host(g.load_frac), to_host(frac)), rep
        assert np.array_equal(to_host(b_graph), to_host(b_eager)), rep
        moved = max(moved, int((to_host(b_graph) != 0).sum()))
    assert moved > 0


def test_graph_with_capacity_dropping_matches_oracle_and_eager():
    """The captured layer with moe_dispatch_capped (capacity int(T*k/E*cf)): every
    replay matches the oracle's capped layer and the eager capped layer bit for
    bit, dropped assignments included."""
    cfg = get_config("decode@T64")
    L = make_layer(cfg)
    d = {k: to_dev(v) for k, v in L.items()}
    cap = moe.moe_capacity(cfg.T, cfg.k, cfg.E, cfg.cf)
    assert cap == oracle.capacity(cfg.T, cfg.k, cfg.E, cfg.cf)
    print(f"\n[gpu] graph with capacity decode@T64 cap={cap}", flush=True)
    g = moe.MoELayerGraph(d["wg"], d["bias"], d["w1"], d["w2"], cfg.k, cfg.T, ws1=d["ws1"],
                          ws2=d["ws2"], capacity_factor=cfg.cf, drop=True)
    dropped = 0
    for rep in range(3):
        Lr = _replay_input(cfg, L, 300 + rep)
        xr = to_dev(Lr["x"])
        out_g = to_host(g.run(xr).clone())
        inv_g = to_host(g.dsp["inv"].clone())
        torch.cuda.synchronize()
        report, _, _ = _check_replay(cfg, Lr, g, keep_cap=cap)
        print(f"[gpu] capped graph replay {rep}: {report}", flush=True)
        r = moe.moe_layer_forward(xr, d["wg"], d["bias"], d["w1"], d["w2"], cfg.k, ws1=d["ws1"],
                                  ws2=d["ws2"], capacity=cap)
        torch.cuda.synchronize()
        assert np.array_equal(inv_g, to_host(r["inv"])), rep
        assert np.array_equal(out_g, to_host(r["out"])), rep
        dropped = max(dropped, int((inv_g < 0).sum()))
    assert dropped > 0

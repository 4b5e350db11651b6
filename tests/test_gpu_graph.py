"""Graph replay of the five calls (decode latency): every replay equals the eager layer.

Several replays with different inputs, with eager work and synchronisations in
between; each replay's output, routing and stats must match an eager run of the
same input bit for bit (same kernels, same order, no atomics).
"""
import numpy as np
import pytest
import torch

import sparse_mixture_experts_05_amd as moe
from synth import MoEConfig, get_config, make_layer, redraw_rows
from tests.parity import to_dev, to_host

pytestmark = pytest.mark.gpu


# decode shapes (small-segment GEMM) and a skewed mid-size layer on the 256x256
# kernel with its planning launch, split over short segments in tile pairs
GRAPH_CASES = ["decode@T1", "decode@T16",
               MoEConfig("graph_big_pairs", T=1024, H=512, E=16, k=4, F=512, Fs=256, bias_amp=2.0)]


@pytest.mark.parametrize("case", GRAPH_CASES, ids=lambda c: c if isinstance(c, str) else c.name)
def test_graph_replays_match_eager(case):
    cfg = get_config(case) if isinstance(case, str) else case
    name = cfg.name
    L = make_layer(cfg)
    d = {k: to_dev(v) for k, v in L.items()}
    print(f"\n[gpu] graph {name}", flush=True)
    g = moe.MoELayerGraph(d["wg"], d["bias"], d["w1"], d["w2"], cfg.k, cfg.T, ws1=d["ws1"],
                          ws2=d["ws2"], capacity_factor=cfg.cf)
    for rep in range(4):
        xr = to_dev(redraw_rows(cfg, np.arange(cfg.T), 100 + rep))
        out_g = to_host(g.run(xr).clone())
        idx_g = to_host(g.idx.clone())
        counts_g = to_host(g.dsp["counts"].clone())
        torch.cuda.synchronize()
        eager = moe.moe_layer_forward(xr, d["wg"], d["bias"], d["w1"], d["w2"], cfg.k,
                                      ws1=d["ws1"], ws2=d["ws2"])
        torch.cuda.synchronize()
        assert np.array_equal(idx_g, to_host(eager["topk_idx"])), rep
        assert np.array_equal(counts_g, to_host(eager["counts"])), rep
        assert np.array_equal(out_g, to_host(eager["out"])), rep


def test_graph_with_bias_feedback_matches_eager_loop():
    """The graph with the dynamic-bias step: each replay routes with the bias the
    previous replay wrote. An eager loop on its own bias copy must give the same
    bias, mean probabilities, load fractions and output after every step."""
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
        xr = to_dev(redraw_rows(cfg, np.arange(cfg.T), 200 + rep))
        out_g = to_host(g.run(xr).clone())
        torch.cuda.synchronize()
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


def test_graph_with_capacity_dropping_matches_eager():
    """The captured layer with moe_dispatch_capped (capacity int(T*k/E*cf)): every
    replay equals the eager capped layer bit for bit, dropped assignments included."""
    cfg = get_config("decode@T64")
    L = make_layer(cfg)
    d = {k: to_dev(v) for k, v in L.items()}
    cap = moe.moe_capacity(cfg.T, cfg.k, cfg.E, cfg.cf)
    print(f"\n[gpu] graph with capacity decode@T64 cap={cap}", flush=True)
    g = moe.MoELayerGraph(d["wg"], d["bias"], d["w1"], d["w2"], cfg.k, cfg.T, ws1=d["ws1"],
                          ws2=d["ws2"], capacity_factor=cfg.cf, drop=True)
    dropped = 0
    for rep in range(3):
        xr = to_dev(redraw_rows(cfg, np.arange(cfg.T), 300 + rep))
        out_g = to_host(g.run(xr).clone())
        inv_g = to_host(g.dsp["inv"].clone())
        torch.cuda.synchronize()
        r = moe.moe_layer_forward(xr, d["wg"], d["bias"], d["w1"], d["w2"], cfg.k, ws1=d["ws1"],
                                  ws2=d["ws2"], capacity=cap)
        torch.cuda.synchronize()
        assert np.array_equal(inv_g, to_host(r["inv"])), rep
        assert np.array_equal(out_g, to_host(r["out"])), rep
        dropped = max(dropped, int((inv_g < 0).sum()))
    assert dropped > 0

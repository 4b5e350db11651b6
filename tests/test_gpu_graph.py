"""Graph replay of the five calls (decode latency): every replay equals the eager layer.

Several replays with different inputs, with eager work and synchronisations in
between; each replay's output, routing and stats must match an eager run of the
same input bit for bit (same kernels, same order, no atomics).
"""
import numpy as np
import pytest
import torch

import sparse_mixture_experts_05_amd as moe
from synth import get_config, make_layer, redraw_rows
from tests.parity import to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["decode@T1", "decode@T16"])
def test_graph_replays_match_eager(name):
    cfg = get_config(name)
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

"""The FFN reading token rows through perm (moe_expert_ffn_gather) against the
dispatch copy followed by moe_expert_ffn: the same rows reach the same kernels,
so ys, ysh and the layer output must agree bit for bit. Covers the three GEMM
kernels (256x256 tiles incl. the split-K tail, the small-segment tiles, fp32),
the shared expert, and capacity dropping (perm defined only on kept rows).
"""
import numpy as np
import pytest
import torch

import sparse_mixture_experts_05_amd as moe
from synth import MoEConfig, get_config, make_layer
from tests.parity import to_dev, to_host

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny_fp32", None),
    (MoEConfig("g_big_ragged", T=1000, H=384, E=16, k=4, F=320, Fs=192, bias_amp=1.5), None),
    (MoEConfig("g_small_E256", T=600, H=256, E=256, k=8, F=128, bias_amp=2.5), None),
    (MoEConfig("g_split_k", T=600, H=256, E=4, k=1, F=8192, Fs=8192, bias_amp=0.5), None),
    (MoEConfig("g_capped", T=700, H=512, E=8, k=2, F=640, bias_amp=1.0), 150),
    ("decode@T16", None),
]


def _name(c):
    cfg, cap = c
    return (cfg if isinstance(cfg, str) else cfg.name) + ("" if cap is None else f"-cap{cap}")


@pytest.mark.parametrize("case", CASES, ids=_name)
def test_gather_ffn_matches_dispatch_copy(case):
    cfg, cap = case
    cfg = get_config(cfg) if isinstance(cfg, str) else cfg
    L = make_layer(cfg)
    d = {k: to_dev(v) for k, v in L.items()}
    print(f"\n[gpu] gather {cfg.name}: T={cfg.T} E={cfg.E} k={cfg.k} F={cfg.F} Fs={cfg.Fs} "
          f"cap={cap}", flush=True)
    fused = moe.moe_layer_forward(d["x"], d["wg"], d["bias"], d["w1"], d["w2"], cfg.k,
                                  ws1=d["ws1"], ws2=d["ws2"], capacity=cap)
    copy = moe.moe_layer_forward(d["x"], d["wg"], d["bias"], d["w1"], d["w2"], cfg.k,
                                 ws1=d["ws1"], ws2=d["ws2"], capacity=cap, fused_gather=False)
    torch.cuda.synchronize()
    assert fused["xs"] is None and copy["xs"] is not None
    for key in ["topk_idx", "counts", "offsets", "inv"]:
        assert np.array_equal(to_host(fused[key]), to_host(copy[key])), key
    n = int(to_host(fused["offsets"])[-1])
    assert np.array_equal(to_host(fused["ys"][:n]), to_host(copy["ys"][:n]))
    if cfg.Fs:
        assert np.array_equal(to_host(fused["ysh"]), to_host(copy["ysh"]))
    assert np.array_equal(to_host(fused["out"]), to_host(copy["out"]))


TIMED = [MoEConfig("t_big", T=700, H=512, E=8, k=2, F=640),            # 256x256 tiles
         MoEConfig("t_split_k", T=600, H=256, E=4, k=1, F=8192, Fs=8192),  # + split-K reduce
         "decode@T1"]                                                       # decode kernel


@pytest.mark.parametrize("cfg", TIMED, ids=lambda c: c if isinstance(c, str) else c.name)
def test_timed_gather_ffn(cfg):
    """moe_expert_ffn_gather_timed gives the bits of moe_expert_ffn_gather and
    records its four events around the two GEMM launches, in order, inside the
    call."""
    cfg = get_config(cfg) if isinstance(cfg, str) else cfg
    L = make_layer(cfg)
    d = {k: to_dev(v) for k, v in L.items()}
    print(f"\n[gpu] timed gather FFN {cfg.name}", flush=True)
    r = moe.moe_layer_forward(d["x"], d["wg"], d["bias"], d["w1"], d["w2"], cfg.k,
                              ws1=d["ws1"], ws2=d["ws2"])
    args = (d["x"], r["perm"], cfg.k, r["offsets"], d["w1"], d["w2"])
    kw = dict(ws1=d["ws1"], ws2=d["ws2"])
    ys0, ysh0 = moe.moe_expert_ffn_gather(*args, **kw)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    ev[0].record()
    ys1, ysh1 = moe.moe_expert_ffn_gather(*args, **kw, gemm_events=ev[1:5])
    ev[5].record()
    torch.cuda.synchronize()
    assert np.array_equal(to_host(ys0), to_host(ys1))
    if cfg.Fs:
        assert np.array_equal(to_host(ysh0), to_host(ysh1))
    gaps = [ev[i].elapsed_time(ev[i + 1]) for i in range(5)]
    assert all(g >= 0 for g in gaps), gaps          # recorded in this order on the stream
    assert gaps[1] > 0 and gaps[3] > 0, gaps        # the up and down GEMM launches
    assert sum(gaps) <= ev[0].elapsed_time(ev[5]) * (1 + 1e-6) + 1e-3

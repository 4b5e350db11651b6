"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every layer, the five full-size workload shapes included, is checked on
every token: routing, dispatch and stats bit for bit, the expert rows ys, the
shared rows ysh and the output over the whole tensor and row by row (the
oracle runs in token chunks). The case name is printed (and flushed) before
each GPU step.
"""
import numpy as np
import pytest

from synth import MoEConfig
from tests.parity import check_layer, run_layer
from tests.support import conditioned_layer

pytestmark = pytest.mark.gpu

SMALL = [
    "tiny_fp32",
    MoEConfig("edge_T1_E1", T=1, H=64, E=1, k=1, F=64),
    MoEConfig("edge_k_eq_E", T=33, H=128, E=4, k=4, F=128, Fs=64, bias_amp=1.0),
    MoEConfig("edge_E256_T3", T=3, H=64, E=256, k=8, F=64),
    MoEConfig("mid_f32", T=130, H=192, E=5, k=3, F=320, Fs=64, dtype="f32", bias_amp=1.0),
    MoEConfig("mid_bf16_big_tiles", T=700, H=512, E=8, k=2, F=640),
    MoEConfig("mid_bf16_small_tiles", T=257, H=512, E=64, k=8, F=256, Fs=256, bias_amp=1.5),
    MoEConfig("ragged_n_bf16", T=1000, H=384, E=16, k=4, F=320, Fs=192, bias_amp=1.5),
    MoEConfig("mid_E256_skew", T=600, H=256, E=256, k=8, F=128, bias_amp=2.5),
    MoEConfig("route_mc2_T8200", T=8200, H=128, E=32, k=2, F=64, bias_amp=1.0),
    MoEConfig("route_bt16_E64", T=2100, H=256, E=64, k=6, F=64, bias_amp=1.0),
    MoEConfig("route_bt64_E12_H192", T=16400, H=192, E=12, k=3, F=64, bias_amp=1.0),
    # two-launch route above T = 2048 (E > 128), ragged expert and token tiles
    MoEConfig("route_two_launch_E200", T=2500, H=256, E=200, k=8, F=64, bias_amp=1.0),
    # big-tile two-launch route: 64 x 128 tiles (E <= 128), 128 x 256 tiles (E > 128)
    MoEConfig("route_big_E128", T=2100, H=512, E=128, k=8, F=64, bias_amp=1.5),
    MoEConfig("route_big_E136", T=3100, H=256, E=136, k=4, F=64, bias_amp=1.0),
    # one-launch route, 16 tokens per workgroup, few experts (panels split over the waves):
    # ragged token tail, a single stage of K panels (H = 512), one expert
    MoEConfig("route_bt16_E16_H2048", T=2500, H=2048, E=16, k=4, F=64, bias_amp=1.0),
    MoEConfig("route_bt16_E4_H512", T=2100, H=512, E=4, k=2, F=64),
    MoEConfig("route_bt16_E1", T=2048, H=2048, E=1, k=1, F=64),
    # down projection with K = 8192 (routed and shared): the last round is split over K
    MoEConfig("split_k_tail", T=600, H=256, E=4, k=1, F=8192, Fs=8192, bias_amp=0.5),
]

FULL = ["mixtral_8x7b", "fine_grained_zipf", "heavy_skew",
        "decode@T1", "decode@T16", "decode@T32", "decode@T64", "decode@T128"]


def _name(c):
    return c if isinstance(c, str) else c.name


@pytest.mark.parametrize("case", SMALL, ids=_name)
def test_small_layer_parity(case):
    cfg, L, redrawn = conditioned_layer(case)
    print(f"\n[gpu] {cfg.name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} F={cfg.F} "
          f"Fs={cfg.Fs} {cfg.dtype} redrawn={redrawn}", flush=True)
    got = run_layer(cfg, L)
    report = check_layer(cfg, L, got)
    print(f"[gpu] {cfg.name}: {report}", flush=True)


@pytest.mark.parametrize("name", FULL)
def test_full_size_parity(name):
    cfg, L, redrawn = conditioned_layer(name)
    print(f"\n[gpu] {cfg.name}: T={cfg.T} E={cfg.E} k={cfg.k} F={cfg.F} Fs={cfg.Fs} "
          f"redrawn={redrawn}", flush=True)
    got = run_layer(cfg, L)
    print(f"[gpu] {cfg.name}: GPU layer done, comparing every token", flush=True)
    report = check_layer(cfg, L, got, progress=True)
    print(f"[gpu] {cfg.name}: {report}", flush=True)


def test_repeat_runs_are_bit_identical():
    """No order-dependent atomics anywhere: two runs give identical bits."""
    cfg, L, _ = conditioned_layer(MoEConfig("repeat", T=1000, H=384, E=16, k=4, F=320, Fs=192,
                                            bias_amp=1.5))
    print(f"\n[gpu] {cfg.name}: two runs", flush=True)
    a = run_layer(cfg, L)
    b = run_layer(cfg, L)
    for key in ["topk_idx", "topk_w", "counts", "offsets", "perm", "inv", "xs", "ys", "ysh", "out"]:
        assert np.array_equal(a[key], b[key]), key

"""Host logic of bench.py (CPU): the algorithmic work behind every reported
fraction, against per-layer totals worked out independently from the layer
definitions, and the one-GPU guard.

Per layer (bf16, b = 2 bytes): route reads x once, Wg and the bias and writes
the ids and weights; the FFN does 4*T*k*H*F + 4*T*H*Fs flops; combine reads the
T*k expert rows, the ids/weights and the shared rows and writes the output.
"""
import os
import subprocess
import sys

import numpy as np

import bench
from synth import get_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_mixtral_shaped_work():
    w = bench.algorithmic_work(get_config("mixtral_8x7b"))
    T, H, E, k, F = 4096, 4096, 8, 2, 14336
    # x (32 MiB) + Wg (64 KiB) + 8 bytes of id and weight per assignment
    assert w["route_bytes"] == 33_554_432 + 65_536 + 65_536
    assert w["ffn_flops"] == 4 * T * k * H * F == 1_924_145_348_608
    # ys (64 MiB) + 8 bytes per assignment + out (32 MiB)
    assert w["combine_bytes"] == 67_108_864 + 65_536 + 33_554_432
    # ids in, perm and inv out, counts and offsets
    assert w["dispatch_bytes"] == 4 * T * k + 8 * T * k + 4 * (2 * E + 1)


def test_fine_grained_and_heavy_skew_work():
    fg = bench.algorithmic_work(get_config("fine_grained_zipf"))
    # shared expert: 4*T*H*Fs flops on top, and its rows in the combine
    assert fg["ffn_flops"] == 4 * 4096 * 8 * 4096 * 1536 + 4 * 4096 * 4096 * 1536
    assert fg["combine_bytes"] == 32768 * 4096 * 2 + 8 * 32768 + 2 * 4096 * 4096 * 2
    assert fg["route_bytes"] == 4096 * 4096 * 2 + 128 * 4096 * 2 + 4 * 128 + 8 * 32768
    hs = bench.algorithmic_work(get_config("heavy_skew"))
    assert hs["route_bytes"] == 16384 * 4096 * 2 + 256 * 4096 * 2 + 4 * 256 + 8 * 131072
    assert hs["ffn_flops"] == 4 * 131072 * 4096 * 1024


def test_capacity_dropping_counts_kept_rows_only():
    cfg = get_config("fine_grained_zipf")
    kept = np.zeros(cfg.E, dtype=np.int64)
    kept[:3] = [100, 50, 1]
    w = bench.algorithmic_work(cfg, kept=kept)
    assert w["ffn_flops"] == 4 * 151 * 4096 * 1536 + 4 * 4096 * 4096 * 1536
    # three live experts' W1 and W2, the shared expert's, the kept rows out, x once in
    assert w["ffn_weight_bytes"] == (2 * 4096 * 1536 * 2 * 3 + 2 * 4096 * 1536 * 2
                                     + 151 * 4096 * 2 + 4096 * 4096 * 2)


def test_gemm_kernel_name_follows_the_launcher_rule():
    assert bench.gemm_kernel_name(get_config("mixtral_8x7b")) == "gemm_bf16_w4_kernel"
    assert bench.gemm_kernel_name(get_config("heavy_skew")) == "gemm_bf16_w4_kernel"
    assert bench.gemm_kernel_name(get_config("decode@T16")) == "gemm_bf16_kernel"
    assert bench.gemm_kernel_name(get_config("tiny_fp32")) == "gemm_f32_kernel"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_repeats_short_samples():
    from synth.workloads import make_layer
    cfg = get_config("tiny_fp32")
    L = make_layer(cfg)
    cb = bench.cpu_baseline(cfg, L, cfg.T, min_seconds=0.3)
    assert cb["seconds"] >= 0.3 and cb["kind"] == "oracle" and cb["cores"] >= 1
    passes = int(cb["sample"].split(" passes")[0])
    assert passes > 1
    assert abs(cb["value"] - passes * cfg.T / cb["seconds"]) <= 1e-9 * cb["value"]
    # the threads it used, the CPU it ran on and where the time went
    assert 1 <= cb["cores"] <= cb["affinity_cpus"] and cb["cpu_model"]
    st = cb["stage_seconds_per_pass"]
    assert set(st) == {"route", "dispatch", "expert_ffn", "combine", "load_stats"}
    assert all(v >= 0 for v in st.values())
    assert sum(st.values()) * passes <= cb["seconds"] * 1.001


def test_roofline_takes_the_gemm_launch_events():
    """kernel_table: with GEMM launch samples, the roofline rate is the flops
    of one launch (half the FFN's) over the mean of the up and down launch
    times; the whole-call rate stays beside it; without them it falls back to
    the call time halved."""
    cfg = get_config("mixtral_8x7b")
    w = bench.algorithmic_work(cfg)
    calls = {n: np.full(4, 0.01) for n in bench.NAMES}
    calls["expert_ffn"] = np.array([1.8, 1.8, 1.8, 1.8])  # ms per FFN call
    gemm = {"gemm_up": np.array([0.9, 0.94]), "gemm_down": np.array([0.8, 0.76])}
    k, achieved, peak = bench.kernel_table(cfg, calls, w, gemm=gemm)
    launch_ms = np.mean([0.9, 0.94, 0.8, 0.76])
    assert np.isclose(achieved, w["ffn_flops"] / 2 / (launch_ms * 1e-3) / 1e12)
    assert np.isclose(k["expert_ffn"]["gemm_launch_ms"]["mean"], launch_ms)
    assert np.isclose(k["expert_ffn"]["TFLOP/s"], w["ffn_flops"] / 1.8e-3 / 1e12)
    assert peak == bench.BF16_PEAK_TFLOPS
    _, fallback, _ = bench.kernel_table(cfg, calls, w)
    assert np.isclose(fallback, w["ffn_flops"] / 1.8e-3 / 1e12)

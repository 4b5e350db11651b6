"""Benchmark of the MoE FFN layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--only]
                    [--warm] [--graph] [--drop] [--no-cpu-baseline]

A step is one pass of the whole layer over one batch: route, dispatch, grouped
expert FFN, combine and load stats (left on the device), all on one stream
with inputs already resident in HBM. W untimed warm-up steps, then exactly K
timed steps between two device synchronisations; HIP events on the launch
stream time every call of every step. Caches are cold: a kernel reading a
1 GiB buffer (more than the 256 MB last-level cache and all L2s) runs before
every timed step, outside the events, and the step time is the event span of
the five calls (--flush-write: a 1 GiB fill kernel instead, which leaves the
last-level cache full of dirty lines). The same K steps are then timed warm,
as a labelled secondary.

Headline workload: the Mixtral-8x7B-shaped layer (T=4096, H=4096, E=8, top-2,
d_ff=14336, bf16 with fp32 accumulation), random weights and inputs from the
seeded generator. Unless --only, the same run also times the fine-grained
(E=128, top-8, shared expert, Zipf bias) and heavy-skew (T=16384, E=256)
layers and the decode sweep (T = 1..128, graph replay). Prints one JSON line:
  value        tokens/s of the headline layer (T / cold step time)
  roofline     the dominant kernel, the bf16 MFMA grouped GEMM (launched twice
               per step: up and down projections, 2*rows*H*F flops each),
               against the dense bf16 MFMA peak of 2500 TFLOP/s; its launches
               are timed with HIP events that the library records right
               before and after each of them on their stream
               (moe_expert_ffn_gather_timed), in steps interleaved with the
               timed ones (event records add work to the stream)
  kernels      per-call average ms (p10 / median / p90 too) and the achieved
               fraction of its roofline; route, dispatch and combine also as a
               fraction of a plain device copy timed in the same run
               (measured_copy_GB/s)
  measured_dense_gemm  the vendor library's bf16 GEMM on the dense problem of
               the same size (context for the MFMA fraction)
  measured_mfma_loop   the bf16 matrix-core rate of a register-only MFMA loop
               (libmoe_probe.so; context for the MFMA fraction)
  warm         the headline layer with warm caches
  workloads    cold and warm summaries of the other 4096+-token layers
  decode       per-T graph-replayed latency (cold and warm) and the FFN's
               weight-read rate
  cpu_baseline the float64 CPU oracle on a bounded sample of the headline layer
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3
CPU_TARGET_S = 15.0
CALIB_BYTES = 512 << 20
PMC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_bf16_mixtral_8x7b_pmc.md")
GEMM_SOURCE = os.path.join(ROOT, "sparse_mixture_experts_05_amd", "csrc", "ffn.hip")


def algorithmic_work(cfg, counts=None, kept=None, fused=True):
    """Bytes / flops each step must move or compute (per call).

    route:    x once + Wg + bias + ids/weights out
    dispatch: ids in, perm + inv out, counts + offsets out; with the row copy
              (fused=False) also x once in and xs out
    ffn:      4*rows*H*F + 4*T*H*Fs flops (the up and down projections);
              bytes: live expert weights, the rows in (x once when the gather
              is fused, else xs) and ys out
    combine:  ys in, inv + weights in, shared rows in, out
    With capacity dropping, kept[e] is expert e's kept rows: rows = sum(kept)
    (xs, the FFN and ys) and an expert is live if it kept a row.
    """
    T, H, E, k, F, Fs = cfg.T, cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs
    b = 2 if cfg.dtype == "bf16" else 4
    assign = T * k
    rows = assign if kept is None else int(kept.sum())
    route = T * H * b + E * H * b + (4 * E if cfg.bias_amp else 0) + 8 * assign
    dispatch = 4 * assign + 8 * assign + 4 * (2 * E + 1)
    if not fused:
        dispatch += T * H * b + rows * H * b
    ffn_flops = 4 * rows * H * F + 4 * T * H * Fs
    if kept is not None:
        live = int((kept > 0).sum())
    else:
        live = E if counts is None else int((counts > 0).sum())
    ffn_bytes = 2 * H * F * b * live + 2 * H * Fs * b + rows * H * b
    ffn_bytes += T * H * b if fused else rows * H * b
    combine = rows * H * b + 8 * assign + (T * H * b if Fs else 0) + T * H * b
    return dict(route_bytes=route, dispatch_bytes=dispatch, ffn_flops=ffn_flops,
                ffn_weight_bytes=ffn_bytes, combine_bytes=combine)


def gemm_kernel_name(cfg):
    """The grouped-GEMM kernel the FFN launches run (the rule of the library's
    launcher: 256x256 tiles once there are 64 rows per expert on average, on
    the 4-wave kernel while every operand buffer is under 4 GiB)."""
    if cfg.dtype != "bf16":
        return "gemm_f32_kernel"
    if cfg.T * cfg.k < 64 * cfg.E:
        return "gemm_bf16_kernel"
    rows = cfg.T * cfg.k
    wide = max(cfg.T * cfg.H, rows * cfg.H, rows * cfg.F, cfg.T * cfg.Fs) * 2 >= 1 << 32
    return "gemm_bf16_big_kernel" if wide else "gemm_bf16_w4_kernel"


def code_sha256(path):
    """SHA-256 of a source file's code: // comments, trailing blanks and empty
    lines removed, so a comment edit does not count as a kernel change."""
    lines = []
    for line in open(path, encoding="utf-8").read().splitlines():
        line = re.sub(r"//.*", "", line).rstrip()
        if line:
            lines.append(line)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def read_traffic():
    """HBM bytes per launch of the dominant kernel from the committed PMC summary,
    or None if missing or if the kernel code changed since it was taken."""
    try:
        text = open(PMC_SUMMARY).read()
    except OSError:
        return None
    m_src = re.search(r"code_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_src and m_b):
        return None
    if code_sha256(GEMM_SOURCE) != m_src.group(1):
        return None
    return float(m_b.group(1))


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo, the field lscpu prints)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(cfg, L, n_tokens, min_seconds=0.0):
    """The oracle as it stands on the first n_tokens tokens of the same layer,
    passes repeated until min_seconds have gone by; each oracle stage is timed
    on its own (route, dispatch, expert FFNs with the shared expert, combine,
    statistics), in the order the oracle's whole-layer function runs them."""
    from threadpoolctl import threadpool_info

    import oracle

    Ls = dict(L)
    Ls["x"] = L["x"][:n_tokens]
    E = np.asarray(L["wg"]).shape[0]
    stages = dict(route=0.0, dispatch=0.0, expert_ffn=0.0, combine=0.0, load_stats=0.0)
    passes = 0
    t0 = time.perf_counter()
    while True:
        t = time.perf_counter()
        idx, w, _, _ = oracle.route(Ls["x"], Ls["wg"], Ls["bias"], cfg.k)
        t1 = time.perf_counter()
        counts, _, _, _, _ = oracle.dispatch(idx, Ls["x"], E)
        t2 = time.perf_counter()
        y = oracle.expert_outputs(Ls["x"], idx, Ls["w1"], Ls["w2"])
        ysh = oracle.shared_outputs(Ls["x"], Ls["ws1"], Ls["ws2"])
        t3 = time.perf_counter()
        oracle.combine(y, w, ysh)
        t4 = time.perf_counter()
        oracle.load_stats(counts, n_tokens, cfg.k, cfg.cf)
        t5 = time.perf_counter()
        for name, a, b in [("route", t, t1), ("dispatch", t1, t2), ("expert_ffn", t2, t3),
                           ("combine", t3, t4), ("load_stats", t4, t5)]:
            stages[name] += b - a
        del y, ysh
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    pool = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    what = f"{passes} passes over " if passes > 1 else ""
    return {"value": passes * n_tokens / dt, "unit": "tokens/s",
            # the oracle's arithmetic runs in the BLAS pool; it cannot use more
            # threads than the process may run on
            "cores": int(min(pool, affinity)), "kind": "oracle",
            "sample": f"{what}the first {n_tokens} of {cfg.T} tokens of the same layer through "
                      f"the whole float64 oracle (route, dispatch, FFN, combine, stats); {dt:.1f} s",
            "affinity_cpus": int(affinity), "blas_threads": int(pool), "cpu_model": cpu_model(),
            "stage_seconds_per_pass": {k: v / passes for k, v in stages.items()},
            "seconds": dt}


def single_thread_baseline(cfg, L, min_seconds=2.0):
    """The oracle on one BLAS thread over a whole small layer (decode T = 1,
    the tiny fp32 layer), passes repeated until min_seconds have gone by."""
    from threadpoolctl import threadpool_limits

    import oracle  # noqa: F401  (its thread pools load first, so the limit reaches them)

    with threadpool_limits(limits=1):
        cb = cpu_baseline(cfg, L, cfg.T, min_seconds=min_seconds)
    cb.pop("seconds")
    return cb


NAMES = ["route", "dispatch", "expert_ffn", "combine", "load_stats"]


class Layer:
    """Device buffers of one workload, allocated once, and its five calls."""

    def __init__(self, cfg, L, moe, torch, copy_gather=False, drop=False):
        import torch as _t  # noqa: F401
        dev = lambda a: None if a is None else (
            torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() if a.dtype == np.uint16
            else torch.from_numpy(a).cuda())
        self.cfg, self.moe, self.torch = cfg, moe, torch
        self.copy_gather = copy_gather
        self.times_gemm = not copy_gather  # moe_expert_ffn_gather_timed
        self.x, self.wg, self.bias = dev(L["x"]), dev(L["wg"]), dev(L["bias"])
        self.w1, self.w2, self.ws1, self.ws2 = dev(L["w1"]), dev(L["w2"]), dev(L["ws1"]), dev(L["ws2"])
        T, H, E, k, F, Fs = cfg.T, cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs
        rows = T * k
        dt_code = 1 if cfg.dtype == "bf16" else 0
        dtype = self.x.dtype
        c = "cuda"
        self.idx = torch.empty((T, k), dtype=torch.int32, device=c)
        self.wts = torch.empty((T, k), dtype=torch.float32, device=c)
        self.dsp = dict(counts=torch.empty(E, dtype=torch.int32, device=c),
                        offsets=torch.empty(E + 1, dtype=torch.int32, device=c),
                        perm=torch.empty(rows, dtype=torch.int32, device=c),
                        inv=torch.empty(rows, dtype=torch.int32, device=c),
                        xs=torch.empty((rows, H), dtype=dtype, device=c) if copy_gather else None)
        self.ws_r = torch.empty(max(1, moe.moe_route_workspace_bytes(T, H, E, k, dt_code)),
                                dtype=torch.uint8, device=c)
        self.ws_d = torch.empty(max(1, moe.moe_dispatch_workspace_bytes(T, E, k)),
                                dtype=torch.uint8, device=c)
        self.ws_f = torch.empty(max(1, moe.moe_expert_ffn_workspace_bytes(rows, T, H, E, F, Fs,
                                                                          dt_code)),
                                dtype=torch.uint8, device=c)
        self.ys = torch.empty((rows, H), dtype=dtype, device=c)
        self.ysh = torch.empty((T, H), dtype=dtype, device=c) if Fs else None
        self.out = torch.empty((T, H), dtype=dtype, device=c)
        from sparse_mixture_experts_05_amd.binding import STATS_BYTES
        self.st = torch.empty(STATS_BYTES, dtype=torch.uint8, device=c)
        self.ovf = torch.empty(E, dtype=torch.int32, device=c)
        self.strag = torch.empty(E, dtype=torch.int32, device=c)
        self.cap = moe.moe_capacity(T, k, E, cfg.cf) if drop else None
        self.stream = torch.cuda.current_stream()

    def step(self, ev=None, gemm_ev=None):
        moe, s, cfg = self.moe, self.stream, self.cfg
        rec = (lambda i: ev[i].record(s)) if ev is not None else (lambda i: None)
        rec(0)
        moe.moe_route(self.x, self.wg, self.bias, cfg.k, topk_idx=self.idx, topk_w=self.wts,
                      ws=self.ws_r, stream=s)
        rec(1)
        moe.moe_dispatch(self.idx, self.x, cfg.E, out=self.dsp, ws=self.ws_d, stream=s,
                         capacity=self.cap)
        rec(2)
        if self.copy_gather:
            moe.moe_expert_ffn(self.dsp["xs"], self.dsp["offsets"], self.w1, self.w2, x=self.x,
                               ws1=self.ws1, ws2=self.ws2, T=cfg.T, ys=self.ys, ysh=self.ysh,
                               ws=self.ws_f, stream=s)
        else:
            moe.moe_expert_ffn_gather(self.x, self.dsp["perm"], cfg.k, self.dsp["offsets"],
                                      self.w1, self.w2, ws1=self.ws1, ws2=self.ws2, ys=self.ys,
                                      ysh=self.ysh, ws=self.ws_f, stream=s, gemm_events=gemm_ev)
        rec(3)
        moe.moe_combine(self.ys, self.dsp["inv"], self.wts, self.ysh, out=self.out, stream=s)
        rec(4)
        moe.moe_load_stats(self.dsp["counts"], cfg.T, cfg.k, cfg.cf, stats=self.st,
                           overflow=self.ovf, straggler_ids=self.strag, stream=s, read_back=False)
        rec(5)

    def graph(self, drop=False):
        return self.moe.MoELayerGraph(self.wg, self.bias, self.w1, self.w2, self.cfg.k, self.cfg.T,
                                      ws1=self.ws1, ws2=self.ws2, capacity_factor=self.cfg.cf,
                                      drop=drop)


class Flush:
    """Evicts the layer's data from the L2s and the 256 MB last-level cache
    before a step, outside the events: one kernel over a 1 GiB buffer.

    "read" (the default) reads the buffer (a max over it), so the caches end
    up holding clean lines of it. "write" fills it instead; the last-level
    cache then holds 256 MB of dirty lines, and their write-backs compete with
    the timed step's first reads (a heavier condition than a preceding layer
    leaves: its writes are its activations, tens of MB)."""

    def __init__(self, torch, mode="read"):
        self.torch = torch
        self.mode = mode
        self.buf = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")

    def __call__(self, s):
        if self.mode == "write":
            self.buf.fill_(s & 0xFF)   # a fill kernel, not a memset
        else:
            self.sink = self.torch.amax(self.buf.view(self.torch.int64))

    def describe(self):
        return ("a 1 GiB fill kernel before every step (dirty last-level cache)" if self.mode == "write"
                else "a kernel reading 1 GiB before every step")


def timed_steps(layer, torch, steps, flush, gemm=False):
    """K timed eager steps with HIP events around every call (on the launch
    stream). With flush, its kernel runs before every step, outside the
    events. With gemm, every timed step is followed by one more step in which
    the library records events right before and after each GEMM launch
    (samples gemm_up, gemm_down): the records add about 4 us each to the
    stream, so they stay out of the timed steps, and the interleaving gives
    both the same conditions; with gemm="only", the GEMM-timed steps alone.
    Returns the per-call samples (ms) of the timed steps, their event spans
    (ms) and the wall time (s) of the whole loop."""
    only = gemm == "only"  # the GEMM-timed steps alone
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    gev = ([[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
           if gemm and layer.times_gemm else None)
    if only and gev is None:
        return {}, None, 0.0
    if gev:
        for g in gev:  # create the HIP events before the timed steps
            for e in g:
                e.record(layer.stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        if not only:
            if flush is not None:
                flush(s)
            layer.step(events[s])
        if gev:
            if flush is not None:
                flush(s)
            layer.step(None, gev[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    samples = {} if only else {
        n: np.array([events[s][i].elapsed_time(events[s][i + 1]) for s in range(steps)])
        for i, n in enumerate(NAMES)}
    if gev:
        samples["gemm_up"] = np.array([g[0].elapsed_time(g[1]) for g in gev])
        samples["gemm_down"] = np.array([g[2].elapsed_time(g[3]) for g in gev])
    spans = None if only else np.array([events[s][0].elapsed_time(events[s][5]) for s in range(steps)])
    return samples, spans, elapsed


def kernel_table(cfg, samples, work, copy_gather=False, gemm=None):
    """Per-call mean / p10 / median / p90 and the fraction of each call's
    roofline; gemm: samples of a pass with the GEMM launches timed."""
    if gemm is not None and "gemm_up" in gemm:  # from a pass of its own
        samples = dict(samples, gemm_up=gemm["gemm_up"], gemm_down=gemm["gemm_down"])
    per = {n: float(samples[n].mean()) for n in NAMES}
    bf16 = cfg.dtype == "bf16"
    peak = BF16_PEAK_TFLOPS if bf16 else FP32_PEAK_TFLOPS
    ffn_ms = per["expert_ffn"]
    # two launches of the same GEMM kernel per step, equal algorithmic flops each
    call_rate = (work["ffn_flops"] / 2) / ((ffn_ms / 2) * 1e-3) / 1e12
    achieved = call_rate
    launch = None
    if "gemm_up" in samples:
        # the kernel's own launches, timed by events the library records
        # around them on their stream (planning and reduce launches outside)
        launch = float(np.concatenate([samples["gemm_up"], samples["gemm_down"]]).mean())
        achieved = (work["ffn_flops"] / 2) / (launch * 1e-3) / 1e12
    k = {
        "route": {"ms": per["route"], "GB/s": work["route_bytes"] / per["route"] / 1e6},
        "dispatch": {"ms": per["dispatch"], "GB/s": work["dispatch_bytes"] / per["dispatch"] / 1e6},
        "expert_ffn": {"ms": ffn_ms, "TFLOP/s": call_rate, "mfma_frac": call_rate / peak,
                       "weight_stream_GB/s": work["ffn_weight_bytes"] / ffn_ms / 1e6},
        "combine": {"ms": per["combine"], "GB/s": work["combine_bytes"] / per["combine"] / 1e6},
        "load_stats": {"ms": per["load_stats"]},
    }
    for n in ["route", "dispatch", "combine"]:
        k[n]["hbm_frac"] = k[n]["GB/s"] / HBM_PEAK_GBS
    k["expert_ffn"]["weight_hbm_frac"] = k["expert_ffn"]["weight_stream_GB/s"] / HBM_PEAK_GBS
    if not copy_gather:
        k["dispatch"]["moves"] = ("ids and indices only (the FFN gathers the token rows "
                                  "through perm), so launch latency bounds it")
    if launch is not None:
        k["expert_ffn"]["gemm_launch_ms"] = {"up": float(samples["gemm_up"].mean()),
                                             "down": float(samples["gemm_down"].mean()),
                                             "mean": launch}
        k["expert_ffn"]["gemm_TFLOP/s"] = achieved
        k["expert_ffn"]["gemm_mfma_frac"] = achieved / peak
    for n in NAMES:
        p10, p50, p90 = np.percentile(samples[n], [10, 50, 90])
        k[n].update(p10_ms=float(p10), median_ms=float(p50), p90_ms=float(p90))
    return k, achieved, peak


def run_workload(name, args, moe, torch, flush, headline=False):
    """Cold-cache (and warm) timing of one workload; returns a result dict."""
    from synth import get_config, make_layer
    cfg = get_config(name)
    print(f"[bench] workload {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    L = make_layer(cfg)
    layer = Layer(cfg, L, moe, torch, copy_gather=args.copy_gather and headline,
                  drop=args.drop and headline)
    print(f"[bench] {cfg.name}: warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        layer.step()
    torch.cuda.synchronize()
    print(f"[bench] {cfg.name}: timing {args.steps} steps, cold caches", file=sys.stderr, flush=True)
    # each cold step is followed by one with the GEMM launches timed (same caches)
    cold, cold_spans, cold_elapsed = timed_steps(layer, torch, args.steps, flush, gemm=True)
    print(f"[bench] {cfg.name}: timing {args.steps} steps, warm caches", file=sys.stderr, flush=True)
    # warm steps back to back (their wall time is the rate), then a pass with
    # the GEMM launches timed
    warm, warm_spans, warm_elapsed = timed_steps(layer, torch, args.steps, None)
    gemm_warm, _, _ = timed_steps(layer, torch, args.steps, None, gemm="only")
    counts = layer.dsp["counts"].cpu().numpy()
    kept = np.diff(layer.dsp["offsets"].cpu().numpy()) if layer.cap is not None else None
    work = algorithmic_work(cfg, counts, kept, fused=not layer.copy_gather)
    res = {"cfg": cfg, "L": L, "layer": layer, "work": work}
    res["cold"] = kernel_table(cfg, cold, work, layer.copy_gather)
    res["warm"] = kernel_table(cfg, warm, work, layer.copy_gather, gemm_warm)
    res["cold_ms"] = float(cold_spans.mean())
    res["warm_ms"] = warm_elapsed * 1e3 / args.steps
    res["cold_spans"] = cold_spans
    res["elapsed_cold"] = cold_elapsed
    return res


def summary(res, which="cold"):
    """Compact per-workload record for the JSON line."""
    cfg = res["cfg"]
    k, achieved, peak = res[which]
    ms = res["cold_ms"] if which == "cold" else res["warm_ms"]
    return {"tokens/s": cfg.T / (ms * 1e-3), "ms_per_step": ms,
            "gemm_TFLOP/s": achieved, "gemm_mfma_frac": achieved / peak,
            "ffn_call_TFLOP/s": k["expert_ffn"]["TFLOP/s"],
            "route_hbm_frac": k["route"]["hbm_frac"], "combine_hbm_frac": k["combine"]["hbm_frac"],
            "kernels_median_ms": {n: k[n]["median_ms"] for n in NAMES}}


def dense_gemm_reference(cfg, torch, reps=10):
    """Context for the MFMA fraction: the vendor library (hipBLASLt through
    torch.nn.functional.linear) on the dense problem of the same size, all
    T*k routed rows as one matrix, with the weights laid out as the layer's
    (rows along K): [rows, H] x [F, H]^T and [rows, F] x [H, F]^T in bf16
    with fp32 accumulation, timed with events after two untimed calls each."""
    import torch.nn.functional as Fn
    rows, H, F = cfg.T * cfg.k, cfg.H, cfg.F
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(rows, H, device="cuda", generator=g).to(torch.bfloat16)
    w1 = (torch.randn(F, H, device="cuda", generator=g) / 64).to(torch.bfloat16)
    w2 = (torch.randn(H, F, device="cuda", generator=g) / 64).to(torch.bfloat16)
    h = Fn.linear(a, w1)
    out = {}
    for name, x, w in [("up", a, w1), ("down", h, w2)]:
        Fn.linear(x, w)
        Fn.linear(x, w)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(reps):
            Fn.linear(x, w)
        ev1.record()
        torch.cuda.synchronize()
        out[name] = ev0.elapsed_time(ev1) / reps
    del a, w1, w2, h
    torch.cuda.empty_cache()
    flops = 2.0 * rows * H * F
    return {"TFLOP/s": 2 * flops / ((out["up"] + out["down"]) * 1e-3) / 1e12,
            "up_ms": out["up"], "down_ms": out["down"],
            "shape": f"[{rows},{H}]x[{F},{H}]^T and [{rows},{F}]x[{H},{F}]^T, bf16, fp32 accumulation",
            "library": "hipBLASLt (torch.nn.functional.linear), warm caches"}


def mfma_loop_reference(torch, blocks=512, iters=20000):
    """Context for the MFMA fraction: the bf16 matrix-core rate with no memory
    traffic (libmoe_probe.so, moe_probe_mfma_bf16: 8 independent 32x32x16
    MFMA chains per wave, two 4-wave workgroups per CU), timed with events
    over three calls after one untimed call."""
    import ctypes
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sparse_mixture_experts_05_amd",
                        "libmoe_probe.so")
    lib = ctypes.CDLL(path)
    lib.moe_probe_mfma_bf16.restype = ctypes.c_int
    lib.moe_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.moe_probe_mfma_bf16_flops.restype = ctypes.c_double
    lib.moe_probe_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run(n):
        rc = lib.moe_probe_mfma_bf16(blocks, n, ctypes.c_void_p(sink.data_ptr()), stream)
        if rc != 0:
            raise RuntimeError(f"moe_probe_mfma_bf16 returned {rc}")

    run(iters // 10)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(3):
        run(iters)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / 3
    if not bool(torch.isfinite(sink).all()):
        raise RuntimeError("moe_probe_mfma_bf16 produced a non-finite sum")
    del sink
    return {"TFLOP/s": lib.moe_probe_mfma_bf16_flops(blocks, iters) / (ms * 1e-3) / 1e12, "ms": ms,
            "kernel": "register-only v_mfma_f32_32x32x16_bf16 loop, no memory traffic"}


def decode_sweep(args, moe, torch, flush):
    """The decode-shaped sweep: per T, graph-replayed layer latency from cold
    caches (a flush before every replay, events around the replay) and warm
    (replays back to back, the weights of the chosen experts left in the
    caches by the previous replay) and, from cold eager steps, the FFN's
    weight-read rate against HBM."""
    from synth import DECODE_TOKENS, get_config, make_layer
    full = get_config("decode")
    print(f"[bench] decode sweep: generating inputs", file=sys.stderr, flush=True)
    L = make_layer(full)
    out = {}
    single = getattr(args, "single_thread", {})
    for T in DECODE_TOKENS:
        cfg = get_config(f"decode@T{T}")
        Lt = dict(L)
        Lt["x"] = L["x"][:T].copy()
        layer = Layer(cfg, Lt, moe, torch)
        for _ in range(args.warmup):
            layer.step()
        steps = max(args.steps, 30)
        cold, _, _ = timed_steps(layer, torch, steps, flush)
        counts = layer.dsp["counts"].cpu().numpy()
        work = algorithmic_work(cfg, counts)
        k, _, _ = kernel_table(cfg, cold, work)
        g = layer.graph()
        g.x.copy_(layer.x)
        for _ in range(args.warmup):
            g.graph.replay()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        for s in range(steps):
            flush(s)
            ev[s][0].record()
            g.graph.replay()
            ev[s][1].record()
        torch.cuda.synchronize()
        lat = np.array([a.elapsed_time(b) for a, b in ev])
        p10, p50, p90 = np.percentile(lat, [10, 50, 90])
        # warm: the same replays without the flush; the host runs ahead, so
        # each replay is queued before the previous one ends
        ev_w = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        for s in range(steps):
            ev_w[s][0].record()
            g.graph.replay()
            ev_w[s][1].record()
        torch.cuda.synchronize()
        warm_p50 = float(np.median([a.elapsed_time(b) for a, b in ev_w]))
        out[f"T{T}"] = {"graph_latency_ms_median": float(p50), "p10_ms": float(p10),
                        "p90_ms": float(p90), "tokens/s": T / (p50 * 1e-3),
                        "graph_latency_warm_ms_median": warm_p50,
                        "eager_kernels_median_ms": {n: k[n]["median_ms"] for n in NAMES},
                        "ffn_weight_GB/s": work["ffn_weight_bytes"] / k["expert_ffn"]["median_ms"] / 1e6,
                        "ffn_weight_hbm_frac": work["ffn_weight_bytes"] / k["expert_ffn"]["median_ms"]
                        / 1e6 / HBM_PEAK_GBS}
        print(f"[bench] decode T={T}: graph latency {p50 * 1e3:.1f} us cold, {warm_p50 * 1e3:.1f} us warm",
              file=sys.stderr, flush=True)
        del g, layer
        torch.cuda.empty_cache()
        if T == 1 and not getattr(args, "no_cpu_baseline", True):
            single["decode@T1"] = single_thread_baseline(cfg, Lt)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mixtral_8x7b")
    ap.add_argument("--cpu-tokens", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", action="store_true",
                    help="the headline workload only (no fine-grained / heavy-skew sub-results, "
                         "no decode sweep)")
    ap.add_argument("--graph", action="store_true",
                    help="headline value from replays of the five calls captured in one HIP graph")
    ap.add_argument("--drop", action="store_true",
                    help="enforce the expert capacity int(T*k/E*cf) on the headline workload: "
                         "dispatch drops the assignments past it (a variant, not the headline layer)")
    ap.add_argument("--warm", action="store_true",
                    help="headline value from warm caches (default: cold, a 1 GiB read kernel "
                         "before every step, outside the per-call events)")
    ap.add_argument("--flush-write", action="store_true",
                    help="cold caches by a 1 GiB fill kernel (leaves the last-level cache dirty) "
                         "instead of a 1 GiB read")
    ap.add_argument("--copy-gather", action="store_true",
                    help="dispatch copies the rows into xs and the FFN reads xs (the default "
                         "FFN reads x through perm: moe_expert_ffn_gather)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with a plain 512 MiB device copy (scales the HBM byte counters)")
    args = ap.parse_args()
    if args.graph and args.copy_gather:
        ap.error("--graph captures the fused-gather layer; --copy-gather is eager only")
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs the MoE layer on one GPU only (no expert parallelism "
              "or collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_mixture_experts_05_amd as moe

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    moe.lib()  # fail loudly if the HIP library is missing
    flush = Flush(torch, "write" if args.flush_write else "read")

    head = run_workload(args.workload, args, moe, torch, flush, headline=True)
    cfg, work, layer = head["cfg"], head["work"], head["layer"]
    T = cfg.T
    kernels, achieved, peak = head["warm" if args.warm else "cold"]
    if args.warm:
        ms_step = head["warm_ms"]
    else:
        # the flush sits outside the per-call events: the step is the event span
        ms_step = head["cold_ms"]
    value = T / (ms_step * 1e-3)
    if args.graph:
        g = layer.graph(drop=args.drop)
        g.x.copy_(layer.x)
        for _ in range(args.warmup):
            g.graph.replay()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for s in range(args.steps):
            if not args.warm:
                flush(s)
            ev[s][0].record()
            g.graph.replay()
            ev[s][1].record()
        torch.cuda.synchronize()
        ms_step = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        value = T / (ms_step * 1e-3)
        del g
    bf16 = cfg.dtype == "bf16"
    result = {
        "metric": "MoE layer tokens/sec at 1 GPU + MFMA util % (FFN) + HBM GB/s (route/dispatch)",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded Gaussian inputs and random-init weights)",
        "config": {"workload": cfg.name, "tokens": T, "hidden": cfg.H, "experts": cfg.E,
                   "top_k": cfg.k, "d_ff": cfg.F, "shared_d_ff": cfg.Fs,
                   "routing_bias_amplitude": cfg.bias_amp, "capacity_factor": cfg.cf,
                   "parallelism": "single GPU", "capacity_dropping": bool(args.drop),
                   "gather": "dispatch copy (xs)" if args.copy_gather else
                             "fused into the FFN (x read through perm)",
                   "launch": "hip graph replay" if args.graph else "eager",
                   "caches": "warm" if args.warm else
                             f"cold: {flush.describe()}, outside the events"},
        "roofline": {"bound": "mfma" if bf16 else "alu", "kernel": gemm_kernel_name(cfg),
                     "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": read_traffic(),
                     "timing": ("the FFN call's event span, halved (--copy-gather)" if layer.copy_gather
                                else "HIP events recorded by the library right before and after each "
                                     "GEMM launch on its stream (moe_expert_ffn_gather_timed), in "
                                     "steps interleaved with the timed ones (one after each, flushed "
                                     "the same way); mean over their up and down launches")},
        "kernels": kernels,
        "mfma_util_pct_ffn": 100.0 * achieved / peak,
        "warm": summary(head, "warm"),
    }
    del head["layer"], layer
    torch.cuda.empty_cache()
    if not args.only:
        subs = {}
        for name in ["fine_grained_zipf", "heavy_skew"]:
            if name == args.workload:
                continue
            r = run_workload(name, args, moe, torch, flush)
            subs[name] = {"cold": summary(r, "cold"), "warm": summary(r, "warm")}
            del r
            torch.cuda.empty_cache()
        result["workloads"] = subs
        args.single_thread = {}
        result["decode"] = decode_sweep(args, moe, torch, flush)
    # Context for the datasheet fractions of the HBM-bound steps: a plain
    # 512 MiB device copy (1 GiB of reads and writes, beyond the last-level
    # cache) timed with events on the same stream; copy_frac = a step's GB/s
    # over it.
    src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(5):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * CALIB_BYTES * 5 / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    del src, dst
    result["measured_copy_GB/s"] = copy_gbs
    for n in ["route", "dispatch", "combine"]:
        kernels[n]["copy_frac"] = kernels[n]["GB/s"] / copy_gbs
    if bf16:
        ref = dense_gemm_reference(cfg, torch)
        result["measured_dense_gemm"] = ref
        result["roofline"]["frac_of_measured_dense_gemm"] = achieved / ref["TFLOP/s"]
        loop = mfma_loop_reference(torch)
        result["measured_mfma_loop"] = loop
        result["roofline"]["frac_of_measured_mfma_loop"] = achieved / loop["TFLOP/s"]
    if args.copy_calibration:
        # a plain device copy of known size: its FETCH_SIZE / WRITE_SIZE
        # readings convert those counters to bytes for the kernels above
        src = torch.ones(CALIB_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        # a first small sample sizes a second one to about CPU_TARGET_S seconds
        L = head["L"]
        n = min(args.cpu_tokens, T)
        print(f"[bench] cpu baseline on {n} tokens", file=sys.stderr, flush=True)
        cb = cpu_baseline(cfg, L, n)
        if cb["seconds"] < CPU_TARGET_S / 2 and n < T:
            # the whole layer when it fits in about twice the target, else a
            # sample sized to the target (the first sample's rate includes
            # fixed costs, so this errs on the short side)
            est_all = cb["seconds"] * T / n
            n2 = T if est_all <= 2 * CPU_TARGET_S else min(T, int(n * CPU_TARGET_S / max(cb["seconds"], 1e-3)))
            print(f"[bench] cpu baseline on {n2} tokens", file=sys.stderr, flush=True)
            # a whole layer that takes under 10 s is run again until 10 s have gone by
            cb = cpu_baseline(cfg, L, n2, min_seconds=10.0 if n2 == T else 0.0)
        cb.pop("seconds")
        # context: the oracle on one thread over two whole small layers
        from synth import get_config as _gc, make_layer as _ml
        single = dict(getattr(args, "single_thread", {}))
        tiny = _gc("tiny_fp32")
        single["tiny_fp32"] = single_thread_baseline(tiny, _ml(tiny))
        cb["single_thread"] = single
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

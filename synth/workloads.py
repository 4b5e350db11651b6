"""Seeded synthetic inputs shaped like the pages' MoE workloads.

This module draws random numbers and nothing else: it holds none of the layer's
arithmetic (no logits, softmax, routing, FFN or statistics). Both the CPU oracle
tests and the HIP path take their inputs from here.

Workload shapes follow the pages:
  * 8 experts, top-2 (Mixtral 8x7B), "lpqz.cn MoE engineering blog", section 2.2;
  * 128 fine-grained experts, top-8, plus one always-on shared expert,
    "hncyxsy.com Kimi K3 fine-grained MoE" article, introduction;
  * 256 routed experts, top-8, Zipf-skewed expert popularity,
    "Kimi K3 专家路由不均衡诊断" (bjdmk.com.cn), sections 1 and 2 (tables of hit
    frequency and max/min load skew);
  * decode batches of 1..128 tokens, the Kimi K3 article's measured-table batch sizes.
Real traffic and trained weights are not available; Gaussian weights and a Zipf
routing bias stand in for them.

Random streams: ``numpy.random.default_rng([seed, tag, sub])`` (PCG64). Tags:
1 = x, 2 = Wg, 3 = W1, 4 = W2, 5 = Ws1, 6 = Ws2, 7 = expert-rank permutation,
8 = x row redraw. ``sub`` is the expert id for W1/W2 (so experts can be drawn
independently, in parallel), 0 otherwise. For a redraw, the stream is
``[seed, 8, token, attempt]``.

Values: standard normal float32 scaled by the standard deviation; "N(0, 1/H)"
is read as variance 1/H, i.e. std 1/sqrt(H) (Wg, W1, Ws1), and 1/sqrt(F) for
W2 (1/sqrt(Fs) for Ws2). bf16 workloads round to bf16 with round-to-nearest-even
and are held as uint16 bit patterns (numpy has no bf16). The Zipf bias is
b_e = -A * s * ln(rank_e) with rank_e = 1 + pi(e) for a seeded permutation pi
(A = amplitude, s = Zipf exponent), computed in float64 and stored as float32.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

TAG_X, TAG_WG, TAG_W1, TAG_W2, TAG_WS1, TAG_WS2, TAG_RANK, TAG_REDRAW = 1, 2, 3, 4, 5, 6, 7, 8

DECODE_TOKENS = (1, 16, 32, 64, 128)


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int            # tokens
    H: int            # hidden size
    E: int            # routed experts
    k: int            # experts per token
    F: int            # d_ff per routed expert
    Fs: int = 0       # d_ff of the always-on shared expert (0 = none)
    dtype: str = "bf16"   # "bf16" or "f32" for activations and weights
    bias_amp: float = 0.0  # Zipf bias amplitude A (0 = no routing bias)
    zipf_s: float = 1.1
    cf: float = 1.25      # capacity factor
    seed: int = 0
    x_rows: int = 0       # rows drawn for x (decode sweep draws 128 and uses a prefix)

    @property
    def rows(self) -> int:
        return self.T * self.k

    def with_tokens(self, T: int) -> "MoEConfig":
        return replace(self, T=T, name=f"{self.name.split('@')[0]}@T{T}")


CONFIGS = {
    # tiny fp32 layer (fp32 everything, no shared expert, no bias)
    "tiny_fp32": MoEConfig("tiny_fp32", T=64, H=256, E=8, k=2, F=512, dtype="f32"),
    # Mixtral-8x7B-shaped layer
    "mixtral_8x7b": MoEConfig("mixtral_8x7b", T=4096, H=4096, E=8, k=2, F=14336),
    # fine-grained, Zipf-skewed, with a shared expert
    "fine_grained_zipf": MoEConfig("fine_grained_zipf", T=4096, H=4096, E=128, k=8, F=1536,
                                   Fs=1536, bias_amp=1.5),
    # decode-shaped sweep; T is one of DECODE_TOKENS (x drawn for 128 rows, prefix used)
    "decode": MoEConfig("decode", T=128, H=4096, E=128, k=8, F=1536, Fs=1536, x_rows=128),
    # heavy skew, large pool
    "heavy_skew": MoEConfig("heavy_skew", T=16384, H=4096, E=256, k=8, F=1024, bias_amp=2.5),
}


def get_config(name: str) -> MoEConfig:
    """``name`` or ``decode@T<n>``."""
    if "@T" in name:
        base, t = name.split("@T")
        return CONFIGS[base].with_tokens(int(t))
    return CONFIGS[name]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # finite values cannot overflow 32 bits here: max finite bits 0x7F7FFFFF (+sign)
    r = (u >> 16) & np.uint32(1)
    r += u
    r += np.uint32(0x7FFF)
    r >>= 16
    out = r.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _draw(cfg: MoEConfig, tag: int, sub, shape, std: float) -> np.ndarray:
    key = [cfg.seed, tag] + (list(sub) if isinstance(sub, (tuple, list)) else [sub])
    a = np.random.default_rng(key).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return f32_to_bf16_bits(a) if cfg.dtype == "bf16" else a


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def zipf_bias(cfg: MoEConfig) -> np.ndarray | None:
    if cfg.bias_amp == 0.0:
        return None
    perm = np.random.default_rng([cfg.seed, TAG_RANK, 0]).permutation(cfg.E)
    rank = 1.0 + perm.astype(np.float64)
    return (-cfg.bias_amp * cfg.zipf_s * np.log(rank)).astype(np.float32)


def make_layer(cfg: MoEConfig, weights: bool = True) -> dict:
    """Draw every input of one layer call.

    Returns a dict of numpy arrays: x [T,H], wg [E,H], w1 [E,F,H], w2 [E,H,F],
    ws1 [Fs,H] / ws2 [H,Fs] (None without a shared expert), bias [E] float32 or None.
    bf16 tensors are uint16 bit patterns; f32 tensors are float32. With
    ``weights=False`` the expert weights are left out (routing-only use).
    """
    H, E, F, Fs = cfg.H, cfg.E, cfg.F, cfg.Fs
    x_rows = max(cfg.x_rows, cfg.T)
    x = _draw(cfg, TAG_X, 0, (x_rows, H), 1.0)[: cfg.T].copy()
    out = {
        "x": x,
        "wg": _draw(cfg, TAG_WG, 0, (E, H), 1.0 / math.sqrt(H)),
        "bias": zipf_bias(cfg),
        "w1": None, "w2": None, "ws1": None, "ws2": None,
    }
    if not weights:
        return out
    dt = np.uint16 if cfg.dtype == "bf16" else np.float32
    w1 = np.empty((E, F, H), dtype=dt)
    w2 = np.empty((E, H, F), dtype=dt)

    def fill(e):
        w1[e] = _draw(cfg, TAG_W1, e, (F, H), 1.0 / math.sqrt(H))
        w2[e] = _draw(cfg, TAG_W2, e, (H, F), 1.0 / math.sqrt(F))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(E)))
    out["w1"], out["w2"] = w1, w2
    if Fs > 0:
        out["ws1"] = _draw(cfg, TAG_WS1, 0, (Fs, H), 1.0 / math.sqrt(H))
        out["ws2"] = _draw(cfg, TAG_WS2, 0, (H, Fs), 1.0 / math.sqrt(Fs))
    return out


def redraw_rows(cfg: MoEConfig, tokens, attempt: int) -> np.ndarray:
    """Fresh x rows for the given token ids, one stream per (token, attempt)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    rows = [_draw(cfg, TAG_REDRAW, (int(t), attempt), (cfg.H,), 1.0) for t in tokens]
    dt = np.uint16 if cfg.dtype == "bf16" else np.float32
    return np.stack(rows).astype(dt, copy=False) if rows else np.empty((0, cfg.H), dtype=dt)

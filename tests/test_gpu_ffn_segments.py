"""Grouped expert FFN on hand-picked segment layouts, through the C ABI
(moe_expert_ffn), against the oracle's expert FFN segment by segment.

The tile schedule of the 256x256 kernel is built on the device from the
offsets alone, so these layouts aim at its corners: empty experts, segments of
1, 255, 256 and 257 rows, rows in several n-blocks of column tiles, every row
in one expert, the largest expert count, the split-K last round (K >= 8192),
the small-segment kernel, whole-K and split over K, and the decode kernel
(16-row blocks, K split over the waves). ys is filled with NaN first, so a
tile that is never computed (or computed twice into the wrong rows) cannot
pass. Every segment must meet the bf16 bar on its own (relative L2 <= 2e-2
against the float64 oracle), and so must every row and the shared expert.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_05_amd as moe
from synth.workloads import bf16_bits_to_f32, f32_to_bf16_bits
from tests.parity import TOL_BF16_REL_L2, to_dev, to_host

pytestmark = pytest.mark.gpu

# name, H, F, Fs, counts per expert (or ("zipf", E, rows, seed))
CASES = [
    ("ragged_nblocks", 256, 2560, 0, [0, 1, 255, 256, 257, 0, 511, 769]),
    ("multiples_of_256", 384, 512, 256, [256, 512, 0, 768, 256, 0, 0, 1024]),
    ("one_hot_expert", 256, 320, 192, [0] * 11 + [1100] + [0] * 4),
    ("e256_skewed_small_tiles", 128, 192, 0, ("zipf", 256, 22000, 7)),
    ("e256_skewed_big_tiles", 128, 192, 64, ("zipf", 256, 60000, 7)),
    ("split_k_tail", 256, 8192, 8192, [300, 0, 129, 40]),
    ("small_segments", 512, 448, 128, [1, 0, 2, 0, 0, 3, 0, 1, 0, 0, 0, 5, 0, 0, 2, 0]),
    # a few rows and long K (the decode kernel: K in 4 slices per workgroup)
    ("small_split_k", 4096, 512, 256, [1, 0, 2, 0, 0, 0, 1, 0]),
    # the decode kernel (at most 2 rows per expert on average) with segments of
    # 16, 17, 33 and 40 rows (several 16-row blocks re-reading one expert's
    # weights), a 107-row shared group (7 blocks); up K = 256 in 4 slices, down
    # K = 320 (shared 192) whole per wave
    ("decode_kernel_blocks", 256, 320, 192, [17, 0, 33, 16, 1, 0, 40] + [0] * 57),
    # the decode kernel with K in 2 slices per workgroup (K = 384, 640)
    ("decode_kernel_two_slices", 384, 640, 0, [3, 0, 1, 16, 0, 2, 0, 0, 0, 0, 1, 0, 0, 0, 0, 5]),
]


def _counts(spec):
    if isinstance(spec, tuple):
        _, E, rows, seed = spec
        rng = np.random.default_rng([seed, 1])
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p = p[rng.permutation(E)]
        p /= p.sum()
        c = rng.multinomial(rows, p)
        c[rng.choice(E, size=E // 4, replace=False)] = 0  # some idle experts
        return c
    return np.asarray(spec, dtype=np.int64)


def _bf16(rng, shape, std):
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_ffn_segments(case):
    name, H, F, Fs, spec = case
    counts = _counts(spec)
    E = len(counts)
    rows = int(counts.sum())
    T = max(rows, 1)  # shared-expert rows (the buffer rows themselves serve as x)
    rng = np.random.default_rng([11, len(name), rows])
    xs = _bf16(rng, (rows, H), 1.0)
    w1 = _bf16(rng, (E, F, H), H ** -0.5)
    w2 = _bf16(rng, (E, H, F), F ** -0.5)
    ws1 = _bf16(rng, (Fs, H), H ** -0.5) if Fs else None
    ws2 = _bf16(rng, (H, Fs), Fs ** -0.5) if Fs else None
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    big = rows >= 64 * E
    print(f"\n[gpu] ffn segments {name}: E={E} rows={rows} H={H} F={F} Fs={Fs} "
          f"{'256x256 tiles' if big else ('decode kernel' if rows <= 2 * E else 'small tiles')} "
          f"max={counts.max()}", flush=True)

    d_xs = to_dev(xs)
    ys = torch.full((rows, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    ysh = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda") if Fs else None
    moe.moe_expert_ffn(d_xs, to_dev(offsets), to_dev(w1), to_dev(w2),
                       x=d_xs if Fs else None, ws1=to_dev(ws1), ws2=to_dev(ws2), T=T,
                       ys=ys, ysh=ysh)
    torch.cuda.synchronize()
    got = bf16_bits_to_f32(to_host(ys)).astype(np.float64)
    assert np.isfinite(got).all(), "rows left unwritten"
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        ref = oracle.expert_ffn(xs[lo:hi], w1[e], w2[e])
        err = np.linalg.norm(got[lo:hi] - ref) / np.linalg.norm(ref)
        rows_err = np.linalg.norm(got[lo:hi] - ref, axis=1) / np.linalg.norm(ref, axis=1)
        assert err <= TOL_BF16_REL_L2 and rows_err.max() <= TOL_BF16_REL_L2, (e, lo, hi, err,
                                                                             rows_err.max())
    if Fs:
        gsh = bf16_bits_to_f32(to_host(ysh)).astype(np.float64)
        ref = oracle.shared_outputs(xs, ws1, ws2)
        assert np.isfinite(gsh).all()
        err = np.linalg.norm(gsh - ref) / np.linalg.norm(ref)
        rows_err = np.linalg.norm(gsh - ref, axis=1) / np.linalg.norm(ref, axis=1)
        assert err <= TOL_BF16_REL_L2 and rows_err.max() <= TOL_BF16_REL_L2, (err, rows_err.max())


def test_ffn_with_an_operand_buffer_past_4_gib():
    """The 4-wave big-tile kernel addresses its operand rows with 32-bit byte
    offsets; a launch whose A buffer reaches 4 GiB takes the 8-wave kernel.
    Here h (131072 rows x F = 16384, bf16) is exactly 4 GiB: the up projection
    runs on the 4-wave kernel, the down projection on the 8-wave one. Rows at
    both ends of the buffer (their h offsets straddle 2^32 bytes) are checked
    one by one against the oracle's expert FFN, and every row must be written."""
    H, F, E = 64, 16384, 2
    counts = np.array([65536, 65536])
    rows = int(counts.sum())
    rng = np.random.default_rng([11, 4, 32])
    xs = _bf16(rng, (rows, H), 1.0)
    w1 = _bf16(rng, (E, F, H), H ** -0.5)
    w2 = _bf16(rng, (E, H, F), F ** -0.5)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    assert rows * F * 2 >= 1 << 32
    print(f"\n[gpu] ffn with a 4 GiB h buffer: E={E} rows={rows} H={H} F={F}", flush=True)
    ys = torch.full((rows, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_expert_ffn(to_dev(xs), to_dev(offsets), to_dev(w1), to_dev(w2), ys=ys)
    torch.cuda.synchronize()
    got = bf16_bits_to_f32(to_host(ys)).astype(np.float64)
    assert np.isfinite(got).all(), "rows left unwritten"
    pick = np.unique(np.concatenate([np.arange(0, 300), np.arange(65400, 65700),
                                     np.arange(rows - 300, rows),
                                     rng.choice(rows, 200, replace=False)]))
    for e in range(E):
        sel = pick[(pick >= offsets[e]) & (pick < offsets[e + 1])]
        ref = oracle.expert_ffn(xs[sel], w1[e], w2[e])
        err = np.linalg.norm(got[sel] - ref) / np.linalg.norm(ref)
        rows_err = np.linalg.norm(got[sel] - ref, axis=1) / np.linalg.norm(ref, axis=1)
        assert err <= TOL_BF16_REL_L2 and rows_err.max() <= TOL_BF16_REL_L2, (e, err, rows_err.max())
    del ys
    torch.cuda.empty_cache()

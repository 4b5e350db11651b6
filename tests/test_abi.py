"""C-ABI checks that need no GPU: symbols, status strings, validation, workspace queries.

Every call here is rejected by host-side validation before any HIP call, so
nothing is launched (the library's contract: arguments are checked first).
"""
import ctypes
import os
import re

import pytest

import sparse_mixture_experts_05_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_five_steps():
    names = declared_functions()
    for n in ["moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_load_stats",
              "moe_dispatch_capped", "moe_bias_update", "moe_status_string", "moe_route_workspace_bytes", "moe_dispatch_workspace_bytes",
              "moe_expert_ffn_workspace_bytes", "moe_expert_ffn_gather"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = moe.lib()
    for name in declared_functions():
        assert hasattr(lib, name), f"libmoe.so does not export {name}"


def test_status_strings():
    for code in [0, -1, -2, -3, -4, -5]:
        assert moe.moe_status_string(code)
    assert moe.moe_status_string(17) == "unknown status"


def test_stats_struct_size():
    from sparse_mixture_experts_05_amd.binding import STATS_BYTES
    assert STATS_BYTES == 9 * 8 + 3 * 8


def test_route_validation():
    L = moe.lib()
    # null pointers
    assert L.moe_route(None, FAKE, None, 4, 64, 8, 2, 1, FAKE, FAKE, None, None, 0, None) == -1
    assert L.moe_route(FAKE, FAKE, None, 4, 64, 8, 2, 1, None, FAKE, None, None, 0, None) == -1
    # bad dtype, non-positive sizes
    assert L.moe_route(FAKE, FAKE, None, 4, 64, 8, 2, 7, FAKE, FAKE, None, None, 0, None) == -1
    assert L.moe_route(FAKE, FAKE, None, 0, 64, 8, 2, 1, FAKE, FAKE, None, None, 0, None) == -1
    assert L.moe_route(FAKE, FAKE, None, 4, 64, 8, 0, 1, FAKE, FAKE, None, None, 0, None) == -1
    # unsupported shapes: E > 256, k > 8, k > E, H % 64, T*k >= 2^31
    assert L.moe_route(FAKE, FAKE, None, 4, 64, 257, 2, 1, FAKE, FAKE, None, None, 0, None) == -2
    assert L.moe_route(FAKE, FAKE, None, 4, 64, 64, 9, 1, FAKE, FAKE, None, None, 0, None) == -2
    assert L.moe_route(FAKE, FAKE, None, 4, 64, 4, 5, 1, FAKE, FAKE, None, None, 0, None) == -2
    assert L.moe_route(FAKE, FAKE, None, 4, 96, 8, 2, 1, FAKE, FAKE, None, None, 0, None) == -2
    assert L.moe_route(FAKE, FAKE, None, 1 << 28, 64, 64, 8, 1, FAKE, FAKE, None, None, 0, None) == -2


def test_route_workspace():
    L = moe.lib()
    # decode-sized batches use the two-launch path and need a workspace for the
    # score tiles; the query also covers the per-workgroup probability sums
    need = L.moe_route_workspace_bytes(16, 4096, 128, 8, 1)
    assert need >= 16 * 128 * 4 + 4 * 128 * 4 and need % 256 == 0
    assert L.moe_route(FAKE, FAKE, None, 16, 4096, 128, 8, 1, FAKE, FAKE, None, None, 0, None) == -3
    assert L.moe_route(FAKE, FAKE, None, 16, 4096, 128, 8, 1, FAKE, FAKE, FAKE, FAKE, need - 1, None) == -3
    # the one-launch path (large batches, E <= 64) only needs it for the mean
    # probabilities: one row of E floats per workgroup of 16 tokens
    rows16 = lambda T, E: -(-(-(-T // 16) * E * 4) // 256) * 256
    assert L.moe_route_workspace_bytes(4096, 4096, 64, 8, 1) == 256 * 64 * 4
    assert L.moe_route_workspace_bytes(64, 256, 8, 2, 0) == 256
    assert L.moe_route(FAKE, FAKE, None, 4096, 4096, 64, 8, 1, FAKE, FAKE, FAKE, None, 0, None) == -3
    assert L.moe_route(FAKE, FAKE, None, 4096, 4096, 64, 8, 1, FAKE, FAKE, FAKE, FAKE,
                       256 * 64 * 4 - 1, None) == -3
    assert L.moe_route_workspace_bytes(16, 4096, 300, 8, 1) == 0
    assert L.moe_route_workspace_bytes(2500, 4096, 64, 8, 1) == rows16(2500, 64)
    # two launches: partial scores [slices][T][E] fp32, then (with the mean
    # probabilities) one row of E floats per select workgroup: 16 tokens from
    # T = 1024 up, else 4. Few tokens, or E > 64 and T < 6144 (big tiles:
    # 64 x 128 for E <= 128, 128 x 256 above, ~256 workgroups)
    al = lambda b: -(-b // 256) * 256
    assert L.moe_route_workspace_bytes(2500, 4096, 256, 8, 1) > 2500 * 256 * 4
    assert L.moe_route_workspace_bytes(4096, 4096, 128, 8, 1) == (al(4 * 4096 * 128 * 4)
                                                                  + al(256 * 128 * 4))
    # below T = 1024 the select keeps 4 tokens per workgroup (2 K slices of the
    # 16 x 64 partial tiles at T = 1000, E = 128)
    assert L.moe_route_workspace_bytes(1000, 4096, 128, 8, 1) == (al(2 * 1000 * 128 * 4)
                                                                  + al(250 * 128 * 4))
    assert L.moe_route_workspace_bytes(5000, 4096, 256, 8, 1) > 5000 * 256 * 4
    # large batches go back to one launch (64 tokens per workgroup at T = 16384)
    assert L.moe_route_workspace_bytes(16384, 4096, 256, 8, 1) == 256 * 256 * 4
    # the partial scores are needed even without the mean probabilities
    assert L.moe_route(FAKE, FAKE, None, 4096, 4096, 128, 8, 1, FAKE, FAKE, None, FAKE,
                       al(4 * 4096 * 128 * 4) - 1, None) == -3
    # fp32 keeps one launch: only the probability rows (16 tokens per row)
    assert L.moe_route_workspace_bytes(4096, 4096, 128, 8, 0) == 256 * 128 * 4


def test_misaligned_rows_are_rejected():
    """Rows and weights are accessed 16 bytes at a time: an address that is not a
    multiple of 16 is an invalid argument, caught before any launch."""
    L = moe.lib()
    ODD = ctypes.c_void_p(0x1004)
    assert L.moe_route(ODD, FAKE, None, 4096, 4096, 8, 2, 1, FAKE, FAKE, None, None, 0, None) == -1
    assert L.moe_route(FAKE, ODD, None, 4096, 4096, 8, 2, 1, FAKE, FAKE, None, None, 0, None) == -1
    need = L.moe_dispatch_workspace_bytes(4096, 128, 8)
    args = [FAKE, FAKE, 4096, 4096, 128, 8, 1, FAKE, FAKE, FAKE, FAKE, ODD]  # xs
    assert L.moe_dispatch(*args, FAKE, need, None) == -1
    rows, T, H, E, F, Fs = 8192, 4096, 4096, 8, 14336, 0
    fneed = L.moe_expert_ffn_workspace_bytes(rows, T, H, E, F, Fs, 1)
    base = [FAKE, FAKE, rows, E, H, F, ODD, FAKE, None, None, None, T, Fs, 1, FAKE, None]  # w1
    assert L.moe_expert_ffn(*base, FAKE, fneed, None) == -1
    assert L.moe_combine(FAKE, FAKE, FAKE, None, 16, 64, 2, 1, ODD, None) == -1


def test_bias_update_validation():
    L = moe.lib()
    f = ctypes.c_float
    assert L.moe_bias_update(None, 8, f(0.01), FAKE, None, None) == -1
    assert L.moe_bias_update(FAKE, 8, f(0.01), None, None, None) == -1
    assert L.moe_bias_update(FAKE, 0, f(0.01), FAKE, None, None) == -1
    assert L.moe_bias_update(FAKE, 8, f(-0.01), FAKE, None, None) == -1
    assert L.moe_bias_update(FAKE, 8, f(float("nan")), FAKE, None, None) == -1
    assert L.moe_bias_update(FAKE, 8, f(float("inf")), FAKE, None, None) == -1
    assert L.moe_bias_update(FAKE, 257, f(0.01), FAKE, None, None) == -2


def test_dispatch_validation_and_workspace():
    L = moe.lib()
    need = L.moe_dispatch_workspace_bytes(4096, 128, 8)
    assert need >= 128 * 16 * 4 and need % 256 == 0
    assert L.moe_dispatch_workspace_bytes(4096, 300, 8) == 0
    # one [E x blocks] int32 table: 64-token blocks for 256 < T <= 4096 and
    # k >= 4, else 256-token blocks (one block up to T = 256)
    al = lambda b: -(-b // 256) * 256
    assert need == al(128 * 64 * 4)
    assert L.moe_dispatch_workspace_bytes(4096, 8, 2) == al(8 * 16 * 4)
    assert L.moe_dispatch_workspace_bytes(257, 128, 4) == al(128 * 5 * 4)
    assert L.moe_dispatch_workspace_bytes(256, 128, 8) == al(128 * 1 * 4)
    assert L.moe_dispatch_workspace_bytes(4097, 128, 8) == al(128 * 17 * 4)
    assert L.moe_dispatch_workspace_bytes(16384, 256, 8) == al(256 * 64 * 4)
    args = [FAKE, FAKE, 4096, 4096, 128, 8, 1, FAKE, FAKE, FAKE, FAKE, FAKE]
    assert L.moe_dispatch(*args, None, need, None) == -3
    assert L.moe_dispatch(*args, FAKE, need - 1, None) == -3
    bad = list(args)
    bad[7] = None
    assert L.moe_dispatch(*bad, FAKE, need, None) == -1
    bad = list(args)
    bad[4] = 0
    assert L.moe_dispatch(*bad, FAKE, need, None) == -1


def test_dispatch_capped_validation():
    L = moe.lib()
    need = L.moe_dispatch_workspace_bytes(4096, 128, 8)
    args = [FAKE, FAKE, 4096, 4096, 128, 8, 320, 1, FAKE, FAKE, FAKE, FAKE, FAKE]
    assert L.moe_dispatch_capped(*args, None, need, None) == -3
    assert L.moe_dispatch_capped(*args, FAKE, need - 1, None) == -3
    bad = list(args)
    bad[6] = -1  # negative capacity
    assert L.moe_dispatch_capped(*bad, FAKE, need, None) == -1
    bad = list(args)
    bad[8] = None  # counts
    assert L.moe_dispatch_capped(*bad, FAKE, need, None) == -1
    bad = list(args)
    bad[4] = 257  # E
    assert L.moe_dispatch_capped(*bad, FAKE, need, None) == -2


def test_capacity_formula_matches_the_statistics():
    """moe_capacity is the library's own C call (the binding holds no formula);
    it must agree with the oracle's capacity and its statistics field."""
    from oracle import capacity, load_stats
    L = moe.lib()
    for T, k, E, cf in [(4096, 2, 8, 1.25), (4096, 8, 128, 1.25), (16384, 8, 256, 1.25),
                        (1, 8, 128, 1.25), (37, 3, 5, 0.7), (64, 2, 8, 1.25),
                        (16, 8, 128, 1.25), (32, 8, 128, 1.25), (128, 8, 128, 1.25),
                        (3, 1, 7, 2.3333333333333335)]:
        want = capacity(T, k, E, cf)
        assert L.moe_capacity(T, k, E, cf) == want
        assert moe.moe_capacity(T, k, E, cf) == want
        assert want == load_stats([T * k] + [0] * (E - 1), T, k, cf)["capacity"]
    # the closed forms of the workloads: int(T*k/E*1.25)
    assert [L.moe_capacity(T, 8, 128, 1.25) for T in (1, 16, 32, 64, 128, 4096)] == \
        [0, 1, 2, 5, 10, 320]
    assert L.moe_capacity(4096, 2, 8, 1.25) == 1280 and L.moe_capacity(16384, 8, 256, 1.25) == 640
    # invalid arguments give -1; a capacity past INT32_MAX is clamped to it
    for args in [(0, 2, 8, 1.25), (4, 0, 8, 1.25), (4, 2, 0, 1.25), (4, 2, 8, 0.0),
                 (4, 2, 8, -1.0), (4, 2, 8, float("nan")), (4, 2, 8, float("inf"))]:
        assert L.moe_capacity(*args) == -1, args
    assert L.moe_capacity(1 << 20, 8, 1, 1e6) == 2 ** 31 - 1
    with pytest.raises(ValueError):
        moe.moe_capacity(4, 2, 8, 0.0)


def test_binding_holds_no_capacity_formula():
    import inspect
    from sparse_mixture_experts_05_amd import binding
    src = inspect.getsource(binding.moe_capacity)
    assert "lib().moe_capacity" in src and "* float(capacity_factor)" not in src


def test_ffn_validation_and_workspace():
    L = moe.lib()
    rows, T, H, E, F, Fs = 32768, 4096, 4096, 128, 1536, 1536
    need = L.moe_expert_ffn_workspace_bytes(rows, T, H, E, F, Fs, 1)
    assert need >= rows * F * 2 + T * Fs * 2
    assert L.moe_expert_ffn_workspace_bytes(rows, T, H, E, 100, Fs, 1) == 0   # F % 64
    assert L.moe_expert_ffn_workspace_bytes(rows, T, 4000, E, F, Fs, 1) == 0  # H % 64
    base = [FAKE, FAKE, rows, E, H, F, FAKE, FAKE, FAKE, FAKE, FAKE, T, Fs, 1, FAKE, FAKE]
    assert L.moe_expert_ffn(*base, FAKE, need - 1, None) == -3
    shared_missing = list(base)
    shared_missing[9] = None  # ws1 missing while Fs > 0
    assert L.moe_expert_ffn(*shared_missing, FAKE, need, None) == -1
    too_many_rows = list(base)
    too_many_rows[2] = T * 8 + 1
    assert L.moe_expert_ffn(*too_many_rows, FAKE, 1 << 40, None) == -2


def test_combine_and_stats_validation():
    L = moe.lib()
    assert L.moe_combine(None, FAKE, FAKE, None, 16, 64, 2, 1, FAKE, None) == -1
    assert L.moe_combine(FAKE, FAKE, FAKE, None, 16, 64, 9, 1, FAKE, None) == -2
    assert L.moe_load_stats(FAKE, 16, 8, 2, 0.0, FAKE, None, FAKE, None) == -1
    assert L.moe_load_stats(FAKE, 16, 8, 2, float("nan"), FAKE, None, FAKE, None) == -1
    assert L.moe_load_stats(FAKE, 16, 8, 2, 1.25, None, None, FAKE, None) == -1
    assert L.moe_load_stats(FAKE, 16, 300, 2, 1.25, FAKE, None, FAKE, None) == -2


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moe.moe_route(x, torch.zeros(8, 64, dtype=torch.bfloat16), None, 2,
                      topk_idx=torch.zeros(4, 2, dtype=torch.int32),
                      topk_w=torch.zeros(4, 2), stream=type("S", (), {"cuda_stream": 0})())


def test_dispatch_without_row_copy_validation():
    """xs = NULL asks for the ranks only (x is then not read and may be NULL);
    a given xs still needs a 16-byte aligned x."""
    L = moe.lib()
    need = L.moe_dispatch_workspace_bytes(4096, 128, 8)
    ODD = ctypes.c_void_p(0x1004)
    # with xs: x is required and aligned
    assert L.moe_dispatch(FAKE, None, 4096, 4096, 128, 8, 1, FAKE, FAKE, FAKE, FAKE, FAKE,
                          FAKE, need, None) == -1
    assert L.moe_dispatch_capped(FAKE, ODD, 4096, 4096, 128, 8, 10, 1, FAKE, FAKE, FAKE, FAKE,
                                 FAKE, FAKE, need, None) == -1
    # without xs the other checks still apply (workspace, sizes, capacity)
    assert L.moe_dispatch(FAKE, None, 4096, 4096, 128, 8, 1, FAKE, FAKE, FAKE, FAKE, None,
                          None, need, None) == -3
    assert L.moe_dispatch(FAKE, None, 4096, 4096, 300, 8, 1, FAKE, FAKE, FAKE, FAKE, None,
                          FAKE, need, None) == -2
    assert L.moe_dispatch_capped(FAKE, None, 4096, 4096, 128, 8, -1, 1, FAKE, FAKE, FAKE, FAKE,
                                 None, FAKE, need, None) == -1


def test_expert_ffn_gather_validation():
    L = moe.lib()
    rows, T, H, E, F, Fs, k = 8192, 4096, 4096, 8, 14336, 0, 2
    need = L.moe_expert_ffn_workspace_bytes(rows, T, H, E, F, Fs, 1)
    ODD = ctypes.c_void_p(0x1004)

    def call(x=FAKE, perm=FAKE, k_=k, rows_=rows, w1=FAKE, ws=FAKE, nbytes=need, Fs_=Fs,
             ws1=None, ysh=None):
        return L.moe_expert_ffn_gather(x, perm, k_, FAKE, rows_, E, H, F, w1, FAKE, ws1, ws1, T,
                                       Fs_, 1, FAKE, ysh, ws, nbytes, None)

    assert call(x=None) == -1
    assert call(perm=None) == -1
    assert call(x=ODD) == -1
    assert call(w1=ODD) == -1
    assert call(k_=0) == -1
    assert call(k_=9) == -2
    assert call(rows_=T * k + 1) == -2      # more rows than assignments
    assert call(ws=None) == -3
    assert call(nbytes=need - 1) == -3
    assert call(Fs_=64) == -1                # shared expert without its weights / output
    assert call(Fs_=64, ws1=FAKE, ysh=ODD) == -1


def test_binding_rejects_mismatched_shapes():
    """The binding checks every tensor's shape (and dtype) before a pointer
    reaches the library: the kernels index by the sizes passed with the
    pointers, so a mismatched tensor would be read or written out of bounds.
    CPU tensors are used: the shape checks come before the device check."""
    import torch
    bf, i32, f32 = torch.bfloat16, torch.int32, torch.float32
    T, H, E, k, F, Fs = 4, 64, 8, 2, 128, 192
    z = lambda *shape, dtype=bf: torch.zeros(*shape, dtype=dtype)
    x, wg = z(T, H), z(E, H)
    idx = z(T, k, dtype=i32)
    w1, w2, ws1, ws2 = z(E, F, H), z(E, H, F), z(Fs, H), z(H, Fs)
    offs = z(E + 1, dtype=i32)
    disp = lambda **kw: dict(dict(counts=z(E, dtype=i32), offsets=offs, perm=z(T * k, dtype=i32),
                                  inv=z(T * k, dtype=i32), xs=z(T * k, H)), **kw)
    cases = {
        "route wg width": lambda: moe.moe_route(x, z(E, H + 64), None, k),
        "route wg dtype": lambda: moe.moe_route(x, z(E, H, dtype=f32), None, k),
        "route bias": lambda: moe.moe_route(x, wg, z(E + 1, dtype=f32), k),
        "route topk_idx": lambda: moe.moe_route(x, wg, None, k, topk_idx=z(T, k + 1, dtype=i32)),
        "route topk_w": lambda: moe.moe_route(x, wg, None, k, topk_w=z(T, k, dtype=torch.float64)),
        "route prob_mean": lambda: moe.moe_route(x, wg, None, k, prob_mean=z(E - 1, dtype=f32)),
        "dispatch ids": lambda: moe.moe_dispatch(z(T + 1, k, dtype=i32), x, E),
        "dispatch counts": lambda: moe.moe_dispatch(idx, x, E, out=disp(counts=z(E + 1, dtype=i32))),
        "dispatch offsets": lambda: moe.moe_dispatch(idx, x, E, out=disp(offsets=z(E, dtype=i32))),
        "dispatch perm": lambda: moe.moe_dispatch(idx, x, E, out=disp(perm=z(T, dtype=i32))),
        "dispatch inv": lambda: moe.moe_dispatch(idx, x, E, out=disp(inv=z(T * k + 1, dtype=i32))),
        "dispatch xs": lambda: moe.moe_dispatch(idx, x, E, out=disp(xs=z(T * k, H + 64))),
        "dispatch capacity": lambda: moe.moe_dispatch(idx, x, E, capacity=-1),
        "ffn offsets": lambda: moe.moe_expert_ffn(z(T * k, H), z(E, dtype=i32), w1, w2),
        "ffn w2 layout": lambda: moe.moe_expert_ffn(z(T * k, H), offs, w1, z(E, F, H)),
        "ffn ws2": lambda: moe.moe_expert_ffn(z(T * k, H), offs, w1, w2, x=x, ws1=ws1,
                                              ws2=z(Fs, H), T=T),
        "ffn ys": lambda: moe.moe_expert_ffn(z(T * k, H), offs, w1, w2, ys=z(T * k - 1, H)),
        "ffn ysh": lambda: moe.moe_expert_ffn(z(T * k, H), offs, w1, w2, x=x, ws1=ws1, ws2=ws2,
                                              T=T, ysh=z(T, H + 64)),
        "gather perm": lambda: moe.moe_expert_ffn_gather(x, z(T * k - 1, dtype=i32), k, offs, w1, w2),
        "gather rows": lambda: moe.moe_expert_ffn_gather(x, z(T * k, dtype=i32), k, offs, w1, w2,
                                                         rows=T * k + 1),
        "gather w1": lambda: moe.moe_expert_ffn_gather(x, z(T * k, dtype=i32), k, offs,
                                                       z(E, F, H + 64), w2),
        "gather ws1": lambda: moe.moe_expert_ffn_gather(x, z(T * k, dtype=i32), k, offs, w1, w2,
                                                        ws1=z(Fs, H + 64), ws2=ws2),
        "combine inv": lambda: moe.moe_combine(z(T * k, H), z(T * k - 1, dtype=i32), z(T, k, dtype=f32)),
        "combine ys": lambda: moe.moe_combine(z(T * k + 1, H), z(T * k, dtype=i32), z(T, k, dtype=f32)),
        "combine ysh": lambda: moe.moe_combine(z(T * k, H), z(T * k, dtype=i32), z(T, k, dtype=f32),
                                               ysh=z(T + 1, H)),
        "combine out": lambda: moe.moe_combine(z(T * k, H), z(T * k, dtype=i32), z(T, k, dtype=f32),
                                               out=z(T, H, dtype=f32)),
        "stats overflow": lambda: moe.moe_load_stats(z(E, dtype=i32), T, k, 1.25,
                                                     overflow=z(E + 1, dtype=i32)),
        "stats stragglers": lambda: moe.moe_load_stats(z(E, dtype=i32), T, k, 1.25,
                                                       straggler_ids=z(E, dtype=torch.int64)),
        "stats buffer": lambda: moe.moe_load_stats(z(E, dtype=i32), T, k, 1.25,
                                                   stats=z(8, dtype=torch.uint8)),
        "bias update": lambda: moe.moe_bias_update(z(E, dtype=i32), z(E - 1, dtype=f32), 0.1),
    }
    for name, call in cases.items():
        with pytest.raises(ValueError) as info:
            call()
        assert "GPU tensor" not in str(info.value), (name, str(info.value))


def test_dispatch_noalloc_validation():
    """moe_dispatch_noalloc: moe_dispatch's checks, and a histogram table
    (E * ceil(T / 256) * 4 bytes, 64-token blocks for 256 < T <= 4096 with
    k >= 4) beyond its fixed 1 MiB scratch is refused with MOE_ERR_SCRATCH,
    all before any HIP call."""
    L = moe.lib()
    f = L.moe_dispatch_noalloc
    assert f(None, None, 16, 64, 8, 2, 1, FAKE, FAKE, FAKE, FAKE, None, None) == -1
    assert f(FAKE, None, 16, 64, 8, 2, 7, FAKE, FAKE, FAKE, FAKE, None, None) == -1
    assert f(FAKE, None, 16, 64, 8, 2, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1  # xs needs x
    assert f(FAKE, None, 16, 64, 300, 2, 1, FAKE, FAKE, FAKE, FAKE, None, None) == -2
    for E in [1, 8, 128, 256]:
        T_max = (1 << 26) // E        # the largest T whose table fits 1 MiB
        assert L.moe_dispatch_workspace_bytes(T_max, E, 1) <= 1 << 20
        assert L.moe_dispatch_workspace_bytes(T_max + 256, E, 1) > 1 << 20
        assert f(FAKE, None, T_max + 256, 64, E, 1, 1, FAKE, FAKE, FAKE, FAKE, None, None) == -5
    assert "scratch" in moe.moe_status_string(-5)


def test_probe_library_exports_and_validates():
    """libmoe_probe.so (bench context only) exports what include/moe_probe.h
    declares, rejects bad arguments before any HIP call and counts its flops."""
    path = os.path.join(os.path.dirname(moe.lib()._name), "libmoe_probe.so")
    lib = ctypes.CDLL(path)
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "moe_probe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))
    assert names == ["moe_probe_mfma_bf16", "moe_probe_mfma_bf16_flops"]
    for n in names:
        assert hasattr(lib, n), f"libmoe_probe.so does not export {n}"
    lib.moe_probe_mfma_bf16.restype = ctypes.c_int
    lib.moe_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    for blocks, iters, sink in [(0, 1, FAKE), (65537, 1, FAKE), (1, 0, FAKE), (1, 1, None)]:
        assert lib.moe_probe_mfma_bf16(blocks, iters, sink, None) == -1
    lib.moe_probe_mfma_bf16_flops.restype = ctypes.c_double
    lib.moe_probe_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    # 4 waves x 8 chains x 32*32*16*2 flops per round
    assert lib.moe_probe_mfma_bf16_flops(3, 5) == 3 * 4 * 5 * 8 * 32768

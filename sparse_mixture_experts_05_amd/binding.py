"""ctypes binding of libmoe.so: argument marshalling only.

Tensors are PyTorch device tensors (memory and streams only); every
computation happens in the library's HIP kernels, enqueued on the current
stream. Missing library or non-GPU tensors raise: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED",
          -3: "MOE_ERR_WORKSPACE", -4: "MOE_ERR_HIP", -5: "MOE_ERR_SCRATCH"}

_vp, _i, _sz, _d = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_double

SIGNATURES = {
    "moe_route": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_route_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "moe_dispatch_workspace_bytes": (_sz, [_i, _i, _i]),
    "moe_dispatch": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_dispatch_capped": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _sz, _vp]),
    "moe_expert_ffn_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "moe_expert_ffn": (_i, [_vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp,
                            _vp, _vp, _sz, _vp]),
    "moe_expert_ffn_gather": (_i, [_vp, _vp, _i, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _i,
                                   _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "moe_expert_ffn_gather_timed": (_i, [_vp, _vp, _i, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp,
                                         _i, _i, _i, _vp, _vp, _vp, _sz, _vp, _vp]),
    "moe_combine": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp]),
    "moe_load_stats": (_i, [_vp, _i, _i, _i, _d, _vp, _vp, _vp, _vp]),
    "moe_bias_update": (_i, [_vp, _i, ctypes.c_float, _vp, _vp, _vp]),
    "moe_capacity": (ctypes.c_int64, [_i, _i, _i, _d]),
    "moe_dispatch_noalloc": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_status_string": (ctypes.c_char_p, [_i]),
}


class MoELoadStats(ctypes.Structure):
    """Mirror of moe_load_stats_t."""
    _fields_ = [(n, ctypes.c_int64) for n in
                ["num_tokens", "assignments", "capacity", "max_load", "min_load", "dropped",
                 "num_stragglers", "gini_num", "gini_den"]] + \
               [(n, ctypes.c_double) for n in ["load_skew_ratio", "gini", "drop_rate"]]


STATS_BYTES = ctypes.sizeof(MoELoadStats)


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({moe_status_string(status)})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (built in-tree); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_mixture_experts_05_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise MoEError(fn, status)


def _dev(t: torch.Tensor | None, name: str, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _want(t, name: str, shape, dtype=None):
    """Shape (and dtype) check of a tensor argument before any pointer reaches
    the library: the kernels index by the sizes passed with the pointers, so a
    mismatched tensor would be read or written out of bounds. None passes."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _dims(t, name: str, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise ValueError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def moe_route_workspace_bytes(T: int, H: int, E: int, k: int, dtype_code: int) -> int:
    return lib().moe_route_workspace_bytes(T, H, E, k, dtype_code)


def moe_route(x, wg, bias, k: int, topk_idx=None, topk_w=None, ws=None, stream=None,
              prob_mean=None):
    """Top-k routing: returns (topk_idx int32 [T,k], topk_w fp32 [T,k]).

    prob_mean: optional fp32 [E] device tensor that receives the mean router
    probability of every expert over the T tokens."""
    T, H = _dims(x, "x", 2)
    E = _dims(wg, "wg", 2)[0]
    _want(wg, "wg", (E, H), x.dtype)
    _want(bias, "bias", (E,), torch.float32)
    _want(topk_idx, "topk_idx", (T, k), torch.int32)
    _want(topk_w, "topk_w", (T, k), torch.float32)
    _want(prob_mean, "prob_mean", (E,), torch.float32)
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    dt = _dtype_code(x)
    nbytes = moe_route_workspace_bytes(T, H, E, k, dt)
    if nbytes > 0:
        ws = _workspace(nbytes, x.device, ws)
    ws_ptr = _dev(ws, "ws") if ws is not None else None
    ws_len = ws.numel() if ws is not None else 0
    _check("moe_route", lib().moe_route(
        _dev(x, "x"), _dev(wg, "wg", x.dtype), _dev(bias, "bias", torch.float32), T, H, E, k, dt,
        _dev(topk_idx, "topk_idx", torch.int32), _dev(topk_w, "topk_w", torch.float32),
        _dev(prob_mean, "prob_mean", torch.float32), ws_ptr, ws_len, _stream(stream)))
    return topk_idx, topk_w


def moe_bias_update(counts, bias, gamma: float, load_frac=None, stream=None):
    """Dynamic routing-bias step in place on ``bias`` (fp32 [E]) from the expert
    counts (int32 [E]); writes the load fractions into ``load_frac`` if given.
    Returns load_frac."""
    E = _dims(counts, "counts", 1)[0]
    _want(counts, "counts", (E,), torch.int32)
    _want(bias, "bias", (E,), torch.float32)
    _want(load_frac, "load_frac", (E,), torch.float32)
    _check("moe_bias_update", lib().moe_bias_update(
        _dev(counts, "counts", torch.int32), E, float(gamma), _dev(bias, "bias", torch.float32),
        _dev(load_frac, "load_frac", torch.float32), _stream(stream)))
    return load_frac


def moe_dispatch_workspace_bytes(T: int, E: int, k: int) -> int:
    return lib().moe_dispatch_workspace_bytes(T, E, k)


def moe_expert_ffn_workspace_bytes(rows, T, H, E, F, Fs, dtype_code) -> int:
    return lib().moe_expert_ffn_workspace_bytes(rows, T, H, E, F, Fs, dtype_code)


def _workspace(nbytes: int, device, ws=None):
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError("workspace too small")
        return ws
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def moe_capacity(T: int, k: int, E: int, capacity_factor: float) -> int:
    """Expert capacity, computed by the library (moe_capacity)."""
    cap = lib().moe_capacity(int(T), int(k), int(E), float(capacity_factor))
    if cap < 0:
        raise ValueError(f"moe_capacity: invalid arguments T={T} k={k} E={E} "
                         f"capacity_factor={capacity_factor}")
    return int(cap)


def moe_dispatch(topk_idx, x, E: int, out=None, ws=None, stream=None, capacity=None,
                 gather: bool = True):
    """Returns dict(counts, offsets, perm, inv, xs). With ``capacity`` (int >= 0)
    each expert keeps its first ``capacity`` assignments (moe_dispatch_capped).
    With ``gather=False`` no rows are copied and xs is None (for
    moe_expert_ffn_gather); a given ``out`` without "xs" (or xs None) does the same."""
    T, H = _dims(x, "x", 2)
    k = _dims(topk_idx, "topk_idx", 2)[1]
    _want(topk_idx, "topk_idx", (T, k), torch.int32)
    if out is not None:
        _want(out.get("counts"), "counts", (E,), torch.int32)
        _want(out.get("offsets"), "offsets", (E + 1,), torch.int32)
        _want(out.get("perm"), "perm", (T * k,), torch.int32)
        _want(out.get("inv"), "inv", (T * k,), torch.int32)
        _want(out.get("xs"), "xs", (T * k, H), x.dtype)
        for key in ["counts", "offsets", "perm", "inv"]:
            if out.get(key) is None:
                raise ValueError(f"out[{key!r}] is required")
    if capacity is not None and not 0 <= int(capacity) < 2 ** 31:
        raise ValueError(f"capacity {capacity} outside [0, 2^31)")
    dev = x.device
    if out is None:
        out = dict(counts=torch.empty(E, dtype=torch.int32, device=dev),
                   offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                   perm=torch.empty(T * k, dtype=torch.int32, device=dev),
                   inv=torch.empty(T * k, dtype=torch.int32, device=dev),
                   xs=torch.empty((T * k, H), dtype=x.dtype, device=dev) if gather else None)
    xs = out.get("xs")
    nbytes = moe_dispatch_workspace_bytes(T, E, k)
    ws = _workspace(nbytes, dev, ws)
    tail = (_dtype_code(x),
            _dev(out["counts"], "counts", torch.int32), _dev(out["offsets"], "offsets", torch.int32),
            _dev(out["perm"], "perm", torch.int32), _dev(out["inv"], "inv", torch.int32),
            _dev(xs, "xs", x.dtype), _dev(ws, "ws"), ws.numel(), _stream(stream))
    if capacity is None:
        _check("moe_dispatch", lib().moe_dispatch(
            _dev(topk_idx, "topk_idx", torch.int32), _dev(x, "x"), T, H, E, k, *tail))
    else:
        _check("moe_dispatch_capped", lib().moe_dispatch_capped(
            _dev(topk_idx, "topk_idx", torch.int32), _dev(x, "x"), T, H, E, k, int(capacity),
            *tail))
    return out


def moe_dispatch_noalloc(topk_idx, x, E: int, out=None, stream=None, gather: bool = True):
    """moe_dispatch on the library's fixed device scratch (no workspace): for
    callers that cannot allocate device memory. The same dict as moe_dispatch;
    ``out`` (preallocated outputs) avoids every allocation here too."""
    T, H = _dims(x, "x", 2)
    k = _dims(topk_idx, "topk_idx", 2)[1]
    _want(topk_idx, "topk_idx", (T, k), torch.int32)
    if out is not None:
        _want(out.get("counts"), "counts", (E,), torch.int32)
        _want(out.get("offsets"), "offsets", (E + 1,), torch.int32)
        _want(out.get("perm"), "perm", (T * k,), torch.int32)
        _want(out.get("inv"), "inv", (T * k,), torch.int32)
        _want(out.get("xs"), "xs", (T * k, H), x.dtype)
        for key in ["counts", "offsets", "perm", "inv"]:
            if out.get(key) is None:
                raise ValueError(f"out[{key!r}] is required")
    dev = x.device
    if out is None:
        out = dict(counts=torch.empty(E, dtype=torch.int32, device=dev),
                   offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                   perm=torch.empty(T * k, dtype=torch.int32, device=dev),
                   inv=torch.empty(T * k, dtype=torch.int32, device=dev),
                   xs=torch.empty((T * k, H), dtype=x.dtype, device=dev) if gather else None)
    _check("moe_dispatch_noalloc", lib().moe_dispatch_noalloc(
        _dev(topk_idx, "topk_idx", torch.int32), _dev(x, "x"), T, H, E, k, _dtype_code(x),
        _dev(out["counts"], "counts", torch.int32), _dev(out["offsets"], "offsets", torch.int32),
        _dev(out["perm"], "perm", torch.int32), _dev(out["inv"], "inv", torch.int32),
        _dev(out.get("xs"), "xs", x.dtype), _stream(stream)))
    return out


def moe_expert_ffn(xs, offsets, w1, w2, x=None, ws1=None, ws2=None, T=None, ys=None, ysh=None,
                   ws=None, stream=None):
    """Returns (ys [rows,H], ysh [T,H] or None)."""
    rows, H = _dims(xs, "xs", 2)
    E, F, _ = _dims(w1, "w1", 3)
    Fs = 0 if ws1 is None else _dims(ws1, "ws1", 2)[0]
    if T is None:
        T = x.shape[0] if x is not None else rows
    _want(offsets, "offsets", (E + 1,), torch.int32)
    _want(w1, "w1", (E, F, H), xs.dtype)
    _want(w2, "w2", (E, H, F), xs.dtype)
    _want(x, "x", (T, H), xs.dtype)
    if Fs > 0:
        if x is None or ws2 is None:
            raise ValueError("the shared expert needs x, ws1 and ws2")
        _want(ws1, "ws1", (Fs, H), xs.dtype)
        _want(ws2, "ws2", (H, Fs), xs.dtype)
        _want(ysh, "ysh", (T, H), xs.dtype)
    _want(ys, "ys", (rows, H), xs.dtype)
    dt = _dtype_code(xs)
    dev = xs.device
    if ys is None:
        ys = torch.empty((rows, H), dtype=xs.dtype, device=dev)
    if Fs > 0 and ysh is None:
        ysh = torch.empty((T, H), dtype=xs.dtype, device=dev)
    nbytes = moe_expert_ffn_workspace_bytes(rows, T, H, E, F, Fs, dt)
    ws = _workspace(nbytes, dev, ws)
    _check("moe_expert_ffn", lib().moe_expert_ffn(
        _dev(xs, "xs"), _dev(offsets, "offsets", torch.int32), rows, E, H, F,
        _dev(w1, "w1", xs.dtype), _dev(w2, "w2", xs.dtype), _dev(x, "x", xs.dtype),
        _dev(ws1, "ws1", xs.dtype), _dev(ws2, "ws2", xs.dtype), T, Fs, dt, _dev(ys, "ys", xs.dtype),
        _dev(ysh, "ysh", xs.dtype) if Fs > 0 else None, _dev(ws, "ws"), ws.numel(),
        _stream(stream)))
    return ys, (ysh if Fs > 0 else None)


def moe_expert_ffn_gather(x, perm, k: int, offsets, w1, w2, ws1=None, ws2=None, rows=None,
                          ys=None, ysh=None, ws=None, stream=None, gemm_events=None):
    """moe_expert_ffn reading routed row p from x[perm[p] // k] (no xs copy).
    Returns (ys [rows,H], ysh [T,H] or None); rows defaults to T*k.
    gemm_events: four torch.cuda.Event (timing enabled) that the library
    records right before and after the up and the down GEMM launches
    (moe_expert_ffn_gather_timed), or None."""
    T, H = _dims(x, "x", 2)
    E, F, _ = _dims(w1, "w1", 3)
    Fs = 0 if ws1 is None else _dims(ws1, "ws1", 2)[0]
    rows = T * k if rows is None else rows
    if not 1 <= rows <= T * k:
        raise ValueError(f"rows {rows} outside [1, T*k = {T * k}]")
    if _dims(perm, "perm", 1)[0] < rows or perm.dtype != torch.int32:
        raise ValueError(f"perm must be int32 with at least rows = {rows} entries")
    _want(offsets, "offsets", (E + 1,), torch.int32)
    _want(w1, "w1", (E, F, H), x.dtype)
    _want(w2, "w2", (E, H, F), x.dtype)
    if Fs > 0:
        if ws2 is None:
            raise ValueError("the shared expert needs ws1 and ws2")
        _want(ws1, "ws1", (Fs, H), x.dtype)
        _want(ws2, "ws2", (H, Fs), x.dtype)
        _want(ysh, "ysh", (T, H), x.dtype)
    _want(ys, "ys", (rows, H), x.dtype)
    dt = _dtype_code(x)
    dev = x.device
    if ys is None:
        ys = torch.empty((rows, H), dtype=x.dtype, device=dev)
    if Fs > 0 and ysh is None:
        ysh = torch.empty((T, H), dtype=x.dtype, device=dev)
    nbytes = moe_expert_ffn_workspace_bytes(rows, T, H, E, F, Fs, dt)
    ws = _workspace(nbytes, dev, ws)
    args = (_dev(x, "x"), _dev(perm, "perm", torch.int32), k, _dev(offsets, "offsets", torch.int32),
            rows, E, H, F, _dev(w1, "w1", x.dtype), _dev(w2, "w2", x.dtype),
            _dev(ws1, "ws1", x.dtype), _dev(ws2, "ws2", x.dtype), T, Fs, dt, _dev(ys, "ys", x.dtype),
            _dev(ysh, "ysh", x.dtype) if Fs > 0 else None, _dev(ws, "ws"), ws.numel(),
            _stream(stream))
    if gemm_events is None:
        _check("moe_expert_ffn_gather", lib().moe_expert_ffn_gather(*args))
    else:
        if len(gemm_events) != 4:
            raise ValueError("gemm_events takes four events (up before / after, down before / after)")
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        handles = (ctypes.c_void_p * 4)()
        for i, ev in enumerate(gemm_events):
            if not ev.cuda_event:
                ev.record(s)  # torch creates the HIP event on its first record
            handles[i] = ev.cuda_event
        _check("moe_expert_ffn_gather_timed", lib().moe_expert_ffn_gather_timed(*args, handles))
    return ys, (ysh if Fs > 0 else None)


def moe_combine(ys, inv, topk_w, ysh=None, out=None, stream=None):
    """Returns out [T,H]."""
    T, k = _dims(topk_w, "topk_w", 2)
    H = _dims(ys, "ys", 2)[1]
    _want(topk_w, "topk_w", (T, k), torch.float32)
    _want(ys, "ys", (T * k, H))
    _want(inv, "inv", (T * k,), torch.int32)
    _want(ysh, "ysh", (T, H), ys.dtype)
    _want(out, "out", (T, H), ys.dtype)
    if out is None:
        out = torch.empty((T, H), dtype=ys.dtype, device=ys.device)
    _check("moe_combine", lib().moe_combine(
        _dev(ys, "ys"), _dev(inv, "inv", torch.int32), _dev(topk_w, "topk_w", torch.float32),
        _dev(ysh, "ysh", ys.dtype), T, H, k, _dtype_code(ys), _dev(out, "out", ys.dtype),
        _stream(stream)))
    return out


def moe_load_stats(counts, T: int, k: int, capacity_factor: float, stats=None, overflow=None,
                   straggler_ids=None, stream=None, read_back: bool = True):
    """Enqueue the diagnostics; with read_back, synchronise and return a dict."""
    E = _dims(counts, "counts", 1)[0]
    _want(counts, "counts", (E,), torch.int32)
    if stats is not None and stats.numel() * stats.element_size() < STATS_BYTES:
        raise ValueError(f"stats must hold at least {STATS_BYTES} bytes")
    _want(overflow, "overflow", (E,), torch.int32)
    _want(straggler_ids, "straggler_ids", (E,), torch.int32)
    dev = counts.device
    if stats is None:
        stats = torch.empty(STATS_BYTES, dtype=torch.uint8, device=dev)
    if overflow is None:
        overflow = torch.empty(E, dtype=torch.int32, device=dev)
    if straggler_ids is None:
        straggler_ids = torch.empty(E, dtype=torch.int32, device=dev)
    _check("moe_load_stats", lib().moe_load_stats(
        _dev(counts, "counts", torch.int32), T, E, k, float(capacity_factor), _dev(stats, "stats"),
        _dev(overflow, "overflow", torch.int32), _dev(straggler_ids, "straggler_ids", torch.int32),
        _stream(stream)))
    if not read_back:
        return dict(stats=stats, overflow=overflow, straggler_ids=straggler_ids)
    return read_stats(stats, overflow, straggler_ids)


def read_stats(stats, overflow, straggler_ids) -> dict:
    """Synchronising copy of moe_load_stats' device outputs into a dict (the
    struct fields, overflow, the straggler ids and the -1 padding after them)."""
    raw = MoELoadStats.from_buffer_copy(bytes(stats.cpu().numpy().tobytes()[:STATS_BYTES]))
    d = {name: getattr(raw, name) for name, _ in MoELoadStats._fields_}
    d["overflow"] = overflow.cpu().tolist()
    ids = straggler_ids.cpu().tolist()
    d["straggler_ids"] = ids[: d["num_stragglers"]]
    d["straggler_tail"] = ids[d["num_stragglers"]:]
    return d


def moe_layer_forward(x, wg, bias, w1, w2, k: int, ws1=None, ws2=None, stream=None,
                      prob_mean=None, capacity=None, fused_gather: bool = True):
    """All five steps on one stream (no host synchronisation). Returns a dict.
    prob_mean (optional fp32 [E]) receives the mean router probabilities;
    capacity (optional int) drops each expert's assignments past it.
    fused_gather (default): dispatch copies no rows and the FFN reads x through
    perm (moe_expert_ffn_gather; xs is None); otherwise dispatch writes xs and
    moe_expert_ffn reads it. Both give bit-identical outputs."""
    E = wg.shape[0]
    idx, w = moe_route(x, wg, bias, k, stream=stream, prob_mean=prob_mean)
    d = moe_dispatch(idx, x, E, stream=stream, capacity=capacity, gather=not fused_gather)
    if fused_gather:
        ys, ysh = moe_expert_ffn_gather(x, d["perm"], k, d["offsets"], w1, w2, ws1=ws1, ws2=ws2,
                                        stream=stream)
    else:
        ys, ysh = moe_expert_ffn(d["xs"], d["offsets"], w1, w2, x=x, ws1=ws1, ws2=ws2,
                                 T=x.shape[0], stream=stream)
    out = moe_combine(ys, d["inv"], w, ysh, stream=stream)
    return dict(topk_idx=idx, topk_w=w, ys=ys, ysh=ysh, out=out, **d)


class MoELayerGraph:
    """The five calls captured once into a HIP graph (torch.cuda.CUDAGraph on ROCm)
    and replayed: one graph launch instead of ~10 kernel launches per layer,
    the decode-latency use of graph replay the lpqz.cn MoE blog describes (its
    section 4.3, graph capture of the per-token MoE inference).

    All buffers are allocated once here; ``run(x)`` copies x into the static
    input buffer and replays. The library never allocates, synchronises or
    clears memory with memset, so its launches are capture-safe.

    With ``drop``, dispatch enforces the expert capacity int(T*k/E*cf)
    (moe_dispatch_capped). With ``bias_gamma`` set (and a bias tensor given),
    every replay also ends
    with the dynamic-bias step on ``bias`` in place and writes the mean router
    probabilities ``prob_mean`` and load fractions ``load_frac``: the next
    replay routes with the updated bias.
    """

    def __init__(self, wg, bias, w1, w2, k: int, T: int, ws1=None, ws2=None,
                 capacity_factor: float = 1.25, bias_gamma: float | None = None,
                 drop: bool = False):
        E, H = wg.shape
        F = w1.shape[1]
        Fs = 0 if ws1 is None else ws1.shape[0]
        dev, dtype = wg.device, wg.dtype
        dt = _dtype_code(wg)
        self.k, self.T, self.cf = k, T, capacity_factor
        self.cap = moe_capacity(T, k, E, capacity_factor) if drop else None
        self.wg, self.bias, self.w1, self.w2, self.ws1, self.ws2 = wg, bias, w1, w2, ws1, ws2
        self.x = torch.zeros((T, H), dtype=dtype, device=dev)
        self.idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.dsp = dict(counts=torch.empty(E, dtype=torch.int32, device=dev),
                        offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                        perm=torch.empty(T * k, dtype=torch.int32, device=dev),
                        inv=torch.empty(T * k, dtype=torch.int32, device=dev),
                        xs=None)  # the FFN reads x through perm
        self.ws_r = torch.empty(max(1, moe_route_workspace_bytes(T, H, E, k, dt)),
                                dtype=torch.uint8, device=dev)
        self.ws_d = torch.empty(max(1, moe_dispatch_workspace_bytes(T, E, k)), dtype=torch.uint8,
                                device=dev)
        self.ws_f = torch.empty(max(1, moe_expert_ffn_workspace_bytes(T * k, T, H, E, F, Fs, dt)),
                                dtype=torch.uint8, device=dev)
        self.ys = torch.empty((T * k, H), dtype=dtype, device=dev)
        self.ysh = torch.empty((T, H), dtype=dtype, device=dev) if Fs else None
        self.out = torch.empty((T, H), dtype=dtype, device=dev)
        self.stats = torch.empty(STATS_BYTES, dtype=torch.uint8, device=dev)
        self.overflow = torch.empty(E, dtype=torch.int32, device=dev)
        self.stragglers = torch.empty(E, dtype=torch.int32, device=dev)
        if bias_gamma is not None and bias is None:
            raise ValueError("bias_gamma needs a bias tensor to update")
        self.gamma = bias_gamma
        self.prob_mean = torch.empty(E, dtype=torch.float32, device=dev) if bias_gamma is not None else None
        self.load_frac = torch.empty(E, dtype=torch.float32, device=dev) if bias_gamma is not None else None
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        saved = None if bias is None else bias.clone()
        with torch.cuda.stream(side):
            self._layer()  # one eager pass on a side stream before capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self._layer()
        torch.cuda.synchronize()
        if saved is not None:
            bias.copy_(saved)  # the warm-up pass must not have moved the bias
            torch.cuda.synchronize()

    def _layer(self):
        moe_route(self.x, self.wg, self.bias, self.k, topk_idx=self.idx, topk_w=self.w,
                  ws=self.ws_r, prob_mean=self.prob_mean)
        moe_dispatch(self.idx, self.x, self.wg.shape[0], out=self.dsp, ws=self.ws_d,
                     capacity=self.cap)
        moe_expert_ffn_gather(self.x, self.dsp["perm"], self.k, self.dsp["offsets"], self.w1,
                              self.w2, ws1=self.ws1, ws2=self.ws2, ys=self.ys, ysh=self.ysh,
                              ws=self.ws_f)
        moe_combine(self.ys, self.dsp["inv"], self.w, self.ysh, out=self.out)
        moe_load_stats(self.dsp["counts"], self.T, self.k, self.cf, stats=self.stats,
                       overflow=self.overflow, straggler_ids=self.stragglers, read_back=False)
        if self.gamma is not None:
            moe_bias_update(self.dsp["counts"], self.bias, self.gamma, load_frac=self.load_frac)

    def run(self, x):
        """Copy x into the static input and replay; returns the static output tensor."""
        self.x.copy_(x)
        self.graph.replay()
        return self.out
